// rgdr_device.h -- device code shared by the decode kernels (rgdr_decode.hip) and the
// long-sequence kernel (rgdr_prefill.hip): buffer descriptors, the kernel argument block,
// per-item index resolution, operand loads and staging, cross-lane sums and the helpers of
// the matrix-core (chunk) form. Not part of the C ABI.
//
// Method: MindSpore Lite API page "lite_boost.ops.recurrent_gated_delta_rule", algorithm
// section and parameter list.
#pragma once

#include "rgdr_common.h"

namespace rgdr {

// Tokens per decode call (the page's decode operator takes at most 8).
constexpr int kMaxT = 8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufWord3 = 0x00020000;  // raw (unformatted) buffer descriptor, gfx9 family
// Cache policy bits of the state stream's buffer loads and stores (2 = nontemporal: the
// state is touched once per call) and of the small operand loads.
#ifndef RGDR_STATE_LOAD_POLICY
#define RGDR_STATE_LOAD_POLICY 2
#endif
#ifndef RGDR_STATE_STORE_POLICY
#define RGDR_STATE_STORE_POLICY 2
#endif
#ifndef RGDR_OPS_LOAD_POLICY
#define RGDR_OPS_LOAD_POLICY 0
#endif
constexpr int kCacheNT = 2;  // nontemporal (streaming)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufWord3);
}

// 16-byte stores carry their whole offset in the vector-register operand, with a zero scalar
// offset. Such a store reads its data registers over more than one cycle, so an instruction
// right after it must not overwrite them yet; the compiler inserts that wait only for stores
// without a scalar-register offset, and on this part the hazard also hits stores with one
// (the late lanes then store what the next instruction wrote). Loads may use either form.
template <int POLICY>
__device__ __forceinline__ void store16(u32x4 v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, POLICY);
}

struct DecodeArgs {
    const uint16_t *q, *k, *v, *beta, *pool;
    const float *g, *gk;
    // Fused gate front end: raw projections [B, T, H_v] (fp32 or fp16) and per-head fp32
    // vectors; g and beta are then computed in the kernel instead of read.
    const void *ga, *gb;
    const float *dt_bias, *dscale;
    uint16_t *out, *pool_out;
    float scale;
    int Hq, Hv, T, Dv, N_slots, ntiles, group, n_items;
    int norm_qk;  // fused front end only: L2-normalise each token's q and k head vector
    int item0;    // first item of this launch (items item0 .. n_items-1)
    // T = 1 wave form: ticks of the constant wall clock (s_memrealtime) each wave waits,
    // counted from its own start, before it writes its tile back; 0 = no wait.
    int hold;
    // Per-token states [B, T, H_v, D_k, D_v] bf16 (the snapshot entries; null otherwise).
    uint16_t *snap;
};

// How an item's g and beta arrive: given (bf16 beta, fp32 g), or computed from raw gate
// projections in fp32 or fp16.
enum GateMode { kGateGiven = 0, kGateF32 = 1, kGateF16 = 2 };

// Element offset of gate entry (b, t, h) in a [B, T, H_v] gate tensor, and the raw load of
// it (lanes whose token is absent aim past the range: zero, no data moved).
__device__ __forceinline__ uint32_t gate_raw(const DecodeArgs &a, const void *base, int gate,
                                             int b, int t, int h, bool present) {
    const uint32_t esz = gate == kGateF16 ? 2u : 4u;
    const auto rs = make_rsrc(static_cast<const char *>(base) + (size_t)b * a.T * a.Hv * esz,
                              (uint32_t)(a.T * a.Hv) * esz);
    const uint32_t off = present ? (uint32_t)(t * a.Hv + h) * esz : 0x7FFFFFF0u;
    return gate == kGateF16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0)
                            : __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
}

// Per-head gate vectors of value head h (every lane loads the same two words).
__device__ __forceinline__ void gate_head(const DecodeArgs &a, int h, float &dt, float &ds) {
    const auto rd = make_rsrc(a.dt_bias, (uint32_t)a.Hv * 4);
    const auto rc = make_rsrc(a.dscale, (uint32_t)a.Hv * 4);
    dt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, h * 4, 0, 0));
    ds = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, h * 4, 0, 0));
}

template <int DK, int TV, int NT, int TMAX = kMaxT>
struct TileShape {
    static constexpr int CPL = 8;         // columns per lane: one 16-byte bf16 vector
    static constexpr int LPR = TV / CPL;  // lanes across one tile row
    static constexpr int RPP = NT / LPR;  // tile rows covered per pass of the NT threads
    static constexpr int R = DK / RPP;    // rows held by each thread
    static_assert(NT % 64 == 0 && 64 % LPR == 0 && DK % RPP == 0 && R >= 1, "tile shape");
    static_assert(LPR == 8 || LPR == 16, "lane reduction handles 64- and 128-wide tiles");
    // Per-thread operand vectors of one item (up to TMAX tokens).
    static constexpr int GKV = (TMAX * DK / 4 + NT - 1) / NT;  // float4 of gk
    static constexpr int KQV = (TMAX * DK / 8 + NT - 1) / NT;  // 8 x bf16 of k (and of q)
    static constexpr int VV = (TMAX * TV / 8 + NT - 1) / NT;   // 8 x bf16 of the v tile
    static_assert(NT >= TMAX, "one thread per token for beta");
    // LDS, in floats. Per token: rows[DK] of (decay, k, scale*q, .) | v[TV] | beta and
    // three scalars of the multi-token form.
    static constexpr int TOK = 4 * DK + TV + 4;
    static constexpr int OPS = TMAX * TOK;  // the operands of all tokens of one item
};

// Workgroups are handed to the device's 8 XCDs (each with its own L2) round-robin by
// workgroup id. Remapped, each XCD works through one contiguous range of items instead, so
// items that share operands (the D_v tiles of one head; value heads that share a query/key
// head) meet in the same L2. A bijection of [0, grid) for any grid size.
#ifndef RGDR_XCD_REMAP
#define RGDR_XCD_REMAP 1
#endif
__device__ __forceinline__ int xcd_item(int blk, int grid) {
    if (!RGDR_XCD_REMAP) return blk;
    constexpr int kXcd = 8;
    const int q = grid / kXcd, r = grid % kXcd, x = blk % kXcd;
    return x * q + (x < r ? x : r) + blk / kXcd;
}

// The per-entry index arrays. They are only read, never written by the kernel; passing them
// as separate restrict-qualified kernel arguments lets the compiler read them with scalar
// loads, which do not count against the vector memory counter the state stream uses.
struct Index {
    const int32_t *__restrict__ lens;
    const int32_t *__restrict__ idx;
    const int32_t *__restrict__ nacc;
};

// Everything about one work item that is uniform across the wave.
struct Item {
    int b, h, hq, tile, slot, L, n;
    bool state;  // a live item whose slot is in range: its state is read and committed
};

__device__ __forceinline__ Item resolve(const DecodeArgs &a, const Index &x, int it) {
    Item m;
    const bool live = it < a.n_items;
    const int itc = live ? it : 0;
    m.tile = itc % a.ntiles;
    const int bh = itc / a.ntiles;
    m.h = bh % a.Hv;
    m.b = bh / a.Hv;
    m.hq = m.h / a.group;  // shared query/key head, floor(h * H_q / H_v)
    m.slot = x.idx[m.b];
    const bool valid = m.slot >= 0 && m.slot < a.N_slots;
    const int L = min(max(x.lens[m.b], 0), a.T);
    m.n = min(max(x.nacc[m.b], 0), L);
    m.state = live && valid;
    m.L = m.state ? L : 0;  // skipped entry (or no item): no tokens, zero output
    return m;
}

// Sum of x over the lanes of this wave that hold the same columns (LPR apart). Every lane
// ends with the same value (each step adds a pair of lanes in both orders, and IEEE
// addition is commutative).
template <int LPR>
__device__ __forceinline__ float colsum(float x) {
    if constexpr (LPR == 8) {
        // row_ror:8 within each 16-lane row pairs lane i with lane i ^ 8
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    }
    {
        // lanes 16-31 <-> 0-15 and 48-63 <-> 32-47: each lane meets lane ^ 16
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    {
        // the two halves of the wave: each lane meets lane ^ 32
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                        false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return x;
}

// Sum of x over aligned groups of N consecutive lanes (N = 8, 16 or 64). Every lane of a group
// ends with the same value, as in colsum. Must be reached by the whole wave.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 8 || N == 16 || N == 64, "group size");
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lane ^ 1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lane ^ 2
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)); // other quad of 8
    if constexpr (N >= 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)); // other 8 of 16
    if constexpr (N == 64) x = colsum<16>(x);
    return x;
}

// Multipliers that L2-normalise a head vector from its sum of squares: 1/||x||, and 0 for an
// all-zero vector (which then stays zero).
__device__ __forceinline__ float inv_norm(float ss) {
    return ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
}

template <int DK, int TV, int NT, int TMAX>
struct Ops {
    using Sh = TileShape<DK, TV, NT, TMAX>;
    f32x4 gk[Sh::GKV];
    uint32_t g[Sh::GKV];  // g, or the raw gate projection a, of this vector's token
    u32x4 k[Sh::KQV], q[Sh::KQV], v[Sh::VV];
    uint32_t beta;        // beta (bf16), or the raw projection b, of token tid
    float dt, ds;         // per-head gate vectors (fused gate only)
};

// Issue the loads of one item's operands. Ranges cover only valid tokens, so padded tokens
// are never read (lanes past the range receive zeros and move no data).
template <int DK, int TV, int NT, int TMAX, int GATE>
__device__ __forceinline__ void load_ops(const DecodeArgs &a, const Item &m,
                                         Ops<DK, TV, NT, TMAX> &o, int tid) {
    using Sh = TileShape<DK, TV, NT, TMAX>;
    const size_t bhT = ((size_t)m.b * a.Hv + m.h) * a.T;
    const uint32_t L = (uint32_t)m.L;
    const auto rgk = make_rsrc(a.gk + bhT * DK, L * DK * 4);
    const auto rg = make_rsrc(a.g + bhT, L * 4);
    const size_t qk0 = ((size_t)m.b * a.Hq + m.hq) * a.T * DK;
    const auto rk = make_rsrc(a.k + qk0, L * DK * 2);
    const auto rq = make_rsrc(a.q + qk0, L * DK * 2);
    const auto rv = make_rsrc(a.v + bhT * a.Dv, L * (uint32_t)a.Dv * 2);
    const auto rb = make_rsrc(a.beta + bhT, L * 2);
#pragma unroll
    for (int j = 0; j < Sh::GKV; ++j) {
        const int e = tid + j * NT;  // float4 index in the [L, DK] block
        o.gk[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rgk, e * 16, 0, 0));
        if constexpr (GATE == kGateGiven)
            o.g[j] = __builtin_amdgcn_raw_buffer_load_b32(rg, (e * 4 / DK) * 4, 0, 0);
        else
            o.g[j] = gate_raw(a, a.ga, GATE, m.b, e * 4 / DK, m.h, e * 4 / DK < m.L);
    }
#pragma unroll
    for (int j = 0; j < Sh::KQV; ++j) {
        const int e = tid + j * NT;  // 8-element index in the [L, DK] block
        o.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, e * 16, 0, 0);
        o.q[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, e * 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < Sh::VV; ++j) {
        const int e = tid + j * NT;
        const int t = e / (TV / 8), c8 = e % (TV / 8);
        o.v[j] = __builtin_amdgcn_raw_buffer_load_b128(
            rv, (uint32_t)((t * a.Dv + m.tile * TV + c8 * 8) * 2), 0, 0);
    }
    if constexpr (GATE == kGateGiven) {
        o.beta = __builtin_amdgcn_raw_buffer_load_b16(rb, tid * 2, 0, 0);
    } else {
        o.beta = gate_raw(a, a.gb, GATE, m.b, tid, m.h, tid < m.L);
        gate_head(a, m.h, o.dt, o.ds);
    }
}

// Element offset of one item's state tile in the pool.
template <int DK, int TV>
__device__ __forceinline__ size_t tile_base(const DecodeArgs &a, const Item &m) {
    return ((size_t)m.slot * a.Hv + m.h) * DK * a.Dv + (size_t)m.tile * TV;
}

// Bytes from the tile's first element to the end of its (slot, head) block.
template <int DK, int TV>
__device__ __forceinline__ uint32_t tile_range(const DecodeArgs &a, const Item &m) {
    return m.state ? (uint32_t)(DK * a.Dv - m.tile * TV) * 2 : 0u;
}

// Cross-lane exchanges. permlane32_swap pairs lane i with lane i ^ 32, permlane16_swap lane
// i with lane i ^ 16 (within each half); the DPP row rotate by 8 pairs lane i with i ^ 8.
__device__ __forceinline__ float2 swap32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));  // (a|b) low, (a|b) high
}
__device__ __forceinline__ float2 swap16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));  // even rows, odd rows
}
__device__ __forceinline__ float lane_xor8(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void split_bf16(float x, uint16_t &hi, uint16_t &lo) {
    hi = f32_to_bf16(x);
    lo = f32_to_bf16(x - bf16_to_f32(hi));  // x - hi is exact in fp32
}

// Element c (0..3) of four packed rows of 4 columns, as one MFMA fragment (rows in k order).
__device__ __forceinline__ s16x4 column_frag(const u32x2 (&w)[4], int c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const int e = c >> 1;
    const uint32_t lo = __builtin_amdgcn_perm(w[1][e], w[0][e], sel);
    const uint32_t hi = __builtin_amdgcn_perm(w[3][e], w[2][e], sel);
    return __builtin_bit_cast(s16x4, make_uint2(lo, hi));
}

// 8-byte state stores take the same form as the 16-byte ones (whole offset in the vector
// operand).
template <int POLICY>
__device__ __forceinline__ void store8(u32x2 v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, POLICY);
}

// The phases below reuse LDS areas under other element types; this keeps the compiler from
// moving an access across a phase boundary (the hardware keeps one wave's LDS accesses in
// order).
__device__ __forceinline__ void lds_phase() { asm volatile("" ::: "memory"); }

// Workgroup barrier that orders LDS only: global loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// lane ^ 4 within each group of 8 lanes: mirror the 8 (lane -> 7 - lane), then reverse each
// 4 (lane -> lane ^ 3).
__device__ __forceinline__ float lane_xor4(float x) {
    const int m = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false);
    return __int_as_float(__builtin_amdgcn_update_dpp(0, m, 0x1B, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
// One halving level of the transposed wave sum: lanes with the level's bit clear keep
// values 0 .. H-1, the others H .. 2H-1, each plus the partner's copy of the same value.
template <int H, typename X>
__device__ __forceinline__ void fold_level(const float (&in)[2 * H], float (&out)[H], bool bit, X xch) {
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const float keep = bit ? in[j + H] : in[j], give = bit ? in[j] : in[j + H];
        out[j] = keep + xch(give);
    }
}
// Sum each of 64 per-lane values over the wave, transposed: lane l ends with the total of
// value l. Partners at each level: lane ^ 32, ^ 16, ^ 8, ^ 4, ^ 2, ^ 1.
__device__ __forceinline__ float wave_sum64_transposed(const float (&v)[64], int lane) {
    float a32[32], a16[16], a8[8], a4[4], a2[2], a1[1];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float2 s = swap32(v[j], v[j + 32]);
        a32[j] = s.x + s.y;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float2 s = swap16(a32[j], a32[j + 16]);
        a16[j] = s.x + s.y;
    }
    fold_level<8>(a16, a8, (lane & 8) != 0, [](float x) { return lane_xor8(x); });
    fold_level<4>(a8, a4, (lane & 4) != 0, [](float x) { return lane_xor4(x); });
    fold_level<2>(a4, a2, (lane & 2) != 0, [](float x) { return lane_xor2(x); });
    fold_level<1>(a2, a1, (lane & 1) != 0, [](float x) { return lane_xor1(x); });
    return a1[0];
}

// Eight bf16 values of two 4-element LDS runs (k slots 0..3, then 4..7).
__device__ __forceinline__ bf16x8 lds_pair8(const uint16_t *p0, const uint16_t *p1) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p0), v = *reinterpret_cast<const uint2 *>(p1);
    return __builtin_bit_cast(bf16x8, u32x4{u.x, u.y, v.x, v.y});
}

// Operand staging of the chunk form (128 threads, D_k = 64 or 128, 128-column tiles).
// Planar per token: the row decays d [8][D_k], k [8][D_k] and scale q [8][D_k], then the
// tile's v [8][128] and beta [8]. Each thread writes whole 16-byte runs of consecutive rows, so the
// stores of a wave fall in distinct LDS banks (an interleaved (d, k, q) record per row
// would put 8 to 16 lanes of every store on one bank). Tokens t >= L come out neutral
// (d = 1, k = q = v = 0): their ranged loads returned zeros, and the fused gate's decay is
// forced to 0 for them.
// After the per-row preparation the d, k and q planes are dead; Y^T [128 columns][kChunkYS]
// then takes their place, so that region is at least that large.
constexpr int kChunkYS = 20;  // floats per Y^T row: 16 values and a pad that spreads LDS banks
template <int DK>
constexpr int chunk_vbase() { return 24 * DK > 128 * kChunkYS ? 24 * DK : 128 * kChunkYS; }
template <int DK>
constexpr int chunk_ops() { return chunk_vbase<DK>() + 8 * 128 + 16; }  // floats, 16-B multiple

template <int DK, int GATE>
__device__ __forceinline__ void chunk_stage_ops(const Ops<DK, 128, 128, kMaxT> &o, float *ob,
                                                float scale, bool norm, int L, int tid) {
    constexpr int NT = 128;
    using Sh = TileShape<DK, 128, NT, kMaxT>;
    constexpr int TV = 128;
    float *sd = ob, *sk = ob + 8 * DK, *sq = ob + 16 * DK, *sv = ob + chunk_vbase<DK>();
    float *sb = sv + 8 * TV;
#pragma unroll
    for (int j = 0; j < Sh::GKV; ++j) {
        const int e = tid + j * NT;
        const int t = e * 4 / DK, i0 = e * 4 % DK;
        if (t >= kMaxT) continue;
        float g;
        if constexpr (GATE == kGateGiven)
            g = __uint_as_float(o.g[j]);
        else
            g = t < L ? o.ds * softplus_fast(gate_value<GATE == kGateF16>(o.g[j]) + o.dt) : 0.f;
        const float eg = __expf(g);
        *reinterpret_cast<f32x4 *>(sd + t * DK + i0) =
            f32x4{eg * __expf(o.gk[j].x), eg * __expf(o.gk[j].y), eg * __expf(o.gk[j].z),
                  eg * __expf(o.gk[j].w)};
    }
#pragma unroll
    for (int j = 0; j < Sh::KQV; ++j) {
        const int e = tid + j * NT;
        const int t = e * 8 / DK, i0 = e * 8 % DK;
        if (t >= kMaxT) continue;  // uniform per 8-lane group; past the last token
        const uint32_t kw[4] = {o.k[j].x, o.k[j].y, o.k[j].z, o.k[j].w};
        const uint32_t qw[4] = {o.q[j].x, o.q[j].y, o.q[j].z, o.q[j].w};
        float ks = 1.f, qs = scale;
        if constexpr (GATE != kGateGiven) {
            if (norm) {  // uniform: the whole wave takes it
                // One token's head vector lies in 16 consecutive, aligned lanes.
                float kss = 0.f, qss = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    kss = fmaf(bf16_lo(kw[w]), bf16_lo(kw[w]), kss);
                    kss = fmaf(bf16_hi(kw[w]), bf16_hi(kw[w]), kss);
                    qss = fmaf(bf16_lo(qw[w]), bf16_lo(qw[w]), qss);
                    qss = fmaf(bf16_hi(qw[w]), bf16_hi(qw[w]), qss);
                }
                ks = inv_norm(group_sum<DK / 8>(kss));
                qs = scale * inv_norm(group_sum<DK / 8>(qss));
            }
        }
        float *kr = sk + t * DK + i0, *qr = sq + t * DK + i0;
        *reinterpret_cast<f32x4 *>(kr) = f32x4{bf16_lo(kw[0]) * ks, bf16_hi(kw[0]) * ks,
                                               bf16_lo(kw[1]) * ks, bf16_hi(kw[1]) * ks};
        *reinterpret_cast<f32x4 *>(kr + 4) = f32x4{bf16_lo(kw[2]) * ks, bf16_hi(kw[2]) * ks,
                                                   bf16_lo(kw[3]) * ks, bf16_hi(kw[3]) * ks};
        *reinterpret_cast<f32x4 *>(qr) = f32x4{bf16_lo(qw[0]) * qs, bf16_hi(qw[0]) * qs,
                                               bf16_lo(qw[1]) * qs, bf16_hi(qw[1]) * qs};
        *reinterpret_cast<f32x4 *>(qr + 4) = f32x4{bf16_lo(qw[2]) * qs, bf16_hi(qw[2]) * qs,
                                                   bf16_lo(qw[3]) * qs, bf16_hi(qw[3]) * qs};
    }
#pragma unroll
    for (int j = 0; j < Sh::VV; ++j) {
        const int e = tid + j * NT;
        const int t = e / (TV / 8), c8 = e % (TV / 8);
        f32x4 *dst = reinterpret_cast<f32x4 *>(sv + t * TV + c8 * 8);
        dst[0] = f32x4{bf16_lo(o.v[j].x), bf16_hi(o.v[j].x), bf16_lo(o.v[j].y), bf16_hi(o.v[j].y)};
        dst[1] = f32x4{bf16_lo(o.v[j].z), bf16_hi(o.v[j].z), bf16_lo(o.v[j].w), bf16_hi(o.v[j].w)};
    }
    if (tid < kMaxT) {
        float bt;
        if constexpr (GATE == kGateGiven)
            bt = bf16_to_f32((uint16_t)o.beta);
        else
            bt = sigmoid_fast(gate_value<GATE == kGateF16>(o.beta));
        sb[tid] = bt;
    }
}

}  // namespace rgdr
