// rgdr_decode.hip -- the recurrent gated-delta-rule decode step on gfx950 (MI355X).
//
// Method: MindSpore Lite API page "lite_boost.ops.recurrent_gated_delta_rule", algorithm
// section (decay, memory read, delta update, output, token by token) and parameter list.
//
// The step is HBM-bound: each (batch entry, value head) pair streams its D_k x D_v bf16
// state in once and out once; everything else is small. Three kernel forms share the
// plumbing below; T and the head sizes decide which one runs.
//
// Wave form (T = 1, every single-token decode). One wave owns one (b, h, 128- or 64-column)
// tile over all D_k rows:
//   * lane (cg, rg) holds 8 consecutive columns (a 16-byte bf16 vector) of the rows rg,
//     rg + RG, ...; a wave-wide load covers RG whole tile rows (1 KiB contiguous at 128
//     columns), with 16-byte nontemporal buffer loads;
//   * the tile stays packed in bf16 registers: the reduction widens it on the fly, the
//     update widens it again, adds k (x) u and packs straight into the commit stores;
//   * the D_k reduction finishes inside the wave (in-lane over the lane's rows, then
//     v_permlane16/32_swap and a DPP row rotate), so waves need no LDS exchange and no
//     barrier and run independently; operands sit in a wave-private LDS area;
//   * one item per wave per launch (a call with more items than resident waves becomes
//     several launches); items past the end and skipped entries use empty buffer ranges
//     (no data moves);
//   * in large launches each wave requests its tile before its operands (small launches:
//     operands first), and every wave holds its commit until the launch's reads could have
//     completed, so that HBM sees a read phase and then a write phase;
//   * 64-column tiles while the call fits one launch of the resident grid with them, else
//     128-column tiles (whole 256-byte rows).
//   Per token, steps 2 and 4 share ONE reduction over D_k. With S' the decayed state,
//   p = S'^T k and r = S'^T (scale q) are reduced together with the scalar k.(scale q);
//   then u = beta (v - p) and o = r + (k.(scale q)) u, which equals S_new^T (scale q), and
//   S_new = S' + k (x) u.
//
// Chunk form (1 < T <= 8 at D_k = 128, 5 <= T <= 8 at D_k = 64 or D_v = 64; where D_v is an
// odd multiple of 64 the last tile is 64 columns wide; decode_chunk_kernel). Two waves own
// one (b, h, 128-column) tile; the item's L tokens are unrolled in closed form (decay
// products, two 8 x 8 Gram matrices, a triangular solve), and the two dense contractions of
// that form run on the matrix cores.
//
// Multi-token form (the other calls with 1 < T <= 8; decode_wave_multi_kernel). One
// wave owns one (b, h, 64- or 128-column) tile and keeps it in fp32 registers across the
// tokens, in a scaled form that leaves three FMAs per element and token; the D_k reduction
// also finishes inside the wave.
//
// All forms: every item issues the same sequence of vector memory instructions whatever
// its lengths and slot (the accesses that must not happen get empty buffer ranges), and the
// per-entry index arrays are read with scalar loads, so the in-order vector-memory counter
// waits never drain the prefetched state. Results are deterministic.
#include <atomic>
#include <cstdlib>

#include "rgdr_device.h"

namespace rgdr {


// Widest tile of the wave form (T = 1): 128 columns (whole 256-byte rows at D_v = 128) when
// D_v and the call's size call for it (decode_entry), or always 64.
#ifndef RGDR_WAVE_TILE_V
#define RGDR_WAVE_TILE_V 128
#endif
// Waves per SIMD the wave forms are compiled for (the register budget).
#ifndef RGDR_WAVE_MIN_WAVES
#define RGDR_WAVE_MIN_WAVES 2
#endif


// Write one item's operands into an LDS operand buffer (decay factors formed here; with the
// fused gate, g and beta are computed here too).
template <int DK, int TV, int NT, int TMAX, int GATE>
__device__ __forceinline__ void stage_ops(const Ops<DK, TV, NT, TMAX> &o, float *ob,
                                          float scale, bool norm, int tid) {
    using Sh = TileShape<DK, TV, NT, TMAX>;
#pragma unroll
    for (int j = 0; j < Sh::GKV; ++j) {
        const int e = tid + j * NT;
        const int t = e * 4 / DK, i0 = e * 4 % DK;
        if (t < TMAX) {
            float g;
            if constexpr (GATE == kGateGiven)
                g = __uint_as_float(o.g[j]);
            else
                g = o.ds * softplus_fast(gate_value<GATE == kGateF16>(o.g[j]) + o.dt);
            const float eg = __expf(g);
            float *row = ob + t * Sh::TOK + 4 * i0;
            row[0] = eg * __expf(o.gk[j].x);
            row[4] = eg * __expf(o.gk[j].y);
            row[8] = eg * __expf(o.gk[j].z);
            row[12] = eg * __expf(o.gk[j].w);
        }
    }
#pragma unroll
    for (int j = 0; j < Sh::KQV; ++j) {
        const int e = tid + j * NT;
        const int t = e * 8 / DK, i0 = e * 8 % DK;
        const uint32_t kw[4] = {o.k[j].x, o.k[j].y, o.k[j].z, o.k[j].w};
        const uint32_t qw[4] = {o.q[j].x, o.q[j].y, o.q[j].z, o.q[j].w};
        float ks = 1.f, qs = scale;
        if constexpr (GATE != kGateGiven) {
            if (norm) {  // uniform: the whole wave takes it
                // One token's head vector lies in DK/8 consecutive, aligned lanes.
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
        if (t < TMAX) {
            float *row = ob + t * Sh::TOK + 4 * i0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                row[8 * w + 1] = bf16_lo(kw[w]) * ks;
                row[8 * w + 5] = bf16_hi(kw[w]) * ks;
                row[8 * w + 2] = bf16_lo(qw[w]) * qs;
                row[8 * w + 6] = bf16_hi(qw[w]) * qs;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < Sh::VV; ++j) {
        const int e = tid + j * NT;
        const int t = e / (TV / 8), c8 = e % (TV / 8);
        if (t < TMAX) {
            f32x4 *dst = reinterpret_cast<f32x4 *>(ob + t * Sh::TOK + 4 * DK + c8 * 8);
            dst[0] = f32x4{bf16_lo(o.v[j].x), bf16_hi(o.v[j].x), bf16_lo(o.v[j].y), bf16_hi(o.v[j].y)};
            dst[1] = f32x4{bf16_lo(o.v[j].z), bf16_hi(o.v[j].z), bf16_lo(o.v[j].w), bf16_hi(o.v[j].w)};
        }
    }
    if (tid < TMAX) {
        float bt;
        if constexpr (GATE == kGateGiven)
            bt = bf16_to_f32((uint16_t)o.beta);
        else
            bt = sigmoid_fast(gate_value<GATE == kGateF16>(o.beta));
        ob[tid * Sh::TOK + 4 * DK + TV] = bt;
    }
}


template <int DK, int TV, int NT>
__device__ __forceinline__ void load_state(const DecodeArgs &a, const Item &m,
                                           u32x4 (&raw)[TileShape<DK, TV, NT>::R], int rg,
                                           int cg) {
    using Sh = TileShape<DK, TV, NT>;
    const auto rs = make_rsrc(a.pool + (m.state ? tile_base<DK, TV>(a, m) : 0),
                              tile_range<DK, TV>(a, m));
#pragma unroll
    for (int r = 0; r < Sh::R; ++r)
        raw[r] = __builtin_amdgcn_raw_buffer_load_b128(
            rs, (uint32_t)(((rg + r * Sh::RPP) * a.Dv + cg * 8) * 2), 0, kCacheNT);
}

// ---------------------------------------------------------------------------------------
// Wave-level form for T = 1: one wave owns one (b, h, TVW-column) tile, all D_k rows, so the
// reduction over D_k finishes inside the wave (in-lane over the lane's rows, then lane
// swaps) with no LDS exchange and no barrier; waves run independently. Lane (cg, rg) holds
// columns cg*8 .. cg*8+7 of rows rg, rg + RG, ... (RW = D_k / RG rows, packed bf16); a
// wave-wide load covers RG consecutive tile rows. Operands are staged in a wave-private LDS
// area (program order within one wave needs no barrier). One item per wave: a call with
// more items than the device holds waves at once is split into launches of the resident
// grid (launch_wave).
// ---------------------------------------------------------------------------------------

// LDS per wave of the T = 1 wave form, in bytes. The operand area needs under 3 KiB; the
// launch requests the rest as padding, which holds each compute unit to eight of these waves
// (160 KiB of LDS), two per SIMD, as many as the register budget RGDR_WAVE_MIN_WAVES is built
// for. With room for a third wave per SIMD, a call with more items than resident waves
// (split into launches of the larger resident grid) streams slower: 98.3 to 100.5 against
// 96.4 us at B = 256, H_v = 32, D = 128. The padding is requested at launch (dynamic LDS),
// not declared in the kernel: declared, it let the compiler schedule for the lower
// occupancy (more registers, a different order) and the same workload took 98.2 us.
constexpr int kWaveLdsBytes = 19968;

// Commit hold of the T = 1 wave form: the read rate its length assumes, in GB/s (HBM's
// streaming read rate on this part for large reads), and a cap on its polls of the clock
// (each poll sleeps 128 cycles). Swept at B = 64 and 256, H_v = 32, D = 128: 6000 GB/s
// 23.3 and 93.4 us, 6250 22.8 and 92.0, 6500 22.8 and 92.3, 6750 23.1 and 93.4, 7000 23.3
// and 94.3, no hold 23.9 and 96.7.
#ifndef RGDR_HOLD_READ_GBPS
#define RGDR_HOLD_READ_GBPS 6400
#endif
constexpr int kHoldMaxPolls = 4096;
// Launches of the T = 1 wave form that read at most this many tile bytes issue their
// operand loads before their tile (see decode_wave_kernel): 16.8 MB launches gained 15%,
// 33.5 MB ones were even, 67 MB ones lost 2%.
constexpr double kOpsFirstBytes = 24.0 * 1024 * 1024;

template <int DK, int TVW>
struct WaveShape {
    static constexpr int LPW = TVW / 8;   // lanes across one tile row
    static constexpr int RG = 64 / LPW;   // row groups in the wave
    static constexpr int RW = DK / RG;    // rows per lane
    static constexpr int RPL = DK / 64;   // operand rows loaded per lane (1 or 2)
    static constexpr int VPL = TVW / 64;  // v values loaded per lane (1 or 2)
    static constexpr int OPS = 4 * DK + TVW;  // (d, k, scale*q, 0) per row | v
    static constexpr int LDS_PAD = kWaveLdsBytes - 4 * OPS;  // dynamic LDS requested at launch
    static_assert(LDS_PAD >= 0, "operand area");
    static_assert(DK == 64 || DK == 128, "D_k");
    static_assert(TVW == 64 || TVW == 128, "tile width");
};

template <int DK>
struct WaveOps {
    float gk[DK / 64];
    uint32_t g;     // g, or the raw gate projection a
    uint32_t k, q;  // DK/64 bf16 values each (low half first)
    uint32_t v;     // TVW/64 bf16 values of the v tile (low half first)
    uint32_t beta;  // beta (bf16), or the raw projection b
    float dt, ds;   // per-head gate vectors (fused gate only)
    bool present;   // the item has its token (L = 1)
};

template <int DK, int TVW, int GATE>
__device__ __forceinline__ void wave_load_ops(const DecodeArgs &a, const Item &m, WaveOps<DK> &o,
                                              int lane) {
    using Sh = WaveShape<DK, TVW>;
    const size_t bh = (size_t)m.b * a.Hv + m.h;  // T = 1
    const uint32_t L = (uint32_t)m.L;          // 0 or 1
    const auto rgk = make_rsrc(a.gk + bh * DK, L * DK * 4);
    const size_t qk0 = ((size_t)m.b * a.Hq + m.hq) * DK;
    const auto rk = make_rsrc(a.k + qk0, L * DK * 2);
    const auto rq = make_rsrc(a.q + qk0, L * DK * 2);
    const auto rv = make_rsrc(a.v + bh * a.Dv, L * (uint32_t)a.Dv * 2);
    const auto rs = make_rsrc(a.g + bh, L * 4);
    const auto rb = make_rsrc(a.beta + bh, L * 2);
    if constexpr (Sh::RPL == 2) {
        const auto g2 = __builtin_amdgcn_raw_buffer_load_b64(rgk, lane * 8, 0, RGDR_OPS_LOAD_POLICY);
        o.gk[0] = __uint_as_float(g2[0]);
        o.gk[1] = __uint_as_float(g2[1]);
        o.k = __builtin_amdgcn_raw_buffer_load_b32(rk, lane * 4, 0, RGDR_OPS_LOAD_POLICY);
        o.q = __builtin_amdgcn_raw_buffer_load_b32(rq, lane * 4, 0, RGDR_OPS_LOAD_POLICY);
    } else {
        o.gk[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rgk, lane * 4, 0, RGDR_OPS_LOAD_POLICY));
        o.k = __builtin_amdgcn_raw_buffer_load_b16(rk, lane * 2, 0, RGDR_OPS_LOAD_POLICY);
        o.q = __builtin_amdgcn_raw_buffer_load_b16(rq, lane * 2, 0, RGDR_OPS_LOAD_POLICY);
    }
    if constexpr (Sh::VPL == 2)
        o.v = __builtin_amdgcn_raw_buffer_load_b32(rv, (uint32_t)((m.tile * TVW + lane * 2) * 2), 0, RGDR_OPS_LOAD_POLICY);
    else
        o.v = __builtin_amdgcn_raw_buffer_load_b16(rv, (uint32_t)((m.tile * TVW + lane) * 2), 0, RGDR_OPS_LOAD_POLICY);
    if constexpr (GATE == kGateGiven) {
        o.g = __builtin_amdgcn_raw_buffer_load_b32(rs, 0, 0, RGDR_OPS_LOAD_POLICY);
        o.beta = __builtin_amdgcn_raw_buffer_load_b16(rb, 0, 0, RGDR_OPS_LOAD_POLICY);
    } else {
        o.g = gate_raw(a, a.ga, GATE, m.b, 0, m.h, m.L > 0);
        o.beta = gate_raw(a, a.gb, GATE, m.b, 0, m.h, m.L > 0);
        gate_head(a, m.h, o.dt, o.ds);
    }
    o.present = m.L > 0;
}

// Stages the rows' (d, k, scale q) and the v tile in the wave's LDS area and returns beta.
// Every lane loaded beta (or b) itself and keeps it in a register: a value that only one
// lane wrote to LDS let the compiler sink its load into that lane's branch, after the
// tile's arrival, which put a memory round trip into the middle of the reduction.
template <int DK, int TVW, int GATE>
__device__ __forceinline__ float wave_stage_ops(const WaveOps<DK> &o, float *ob, float scale,
                                                bool norm, int lane) {
    using Sh = WaveShape<DK, TVW>;
    float g, bt;
    if constexpr (GATE == kGateGiven) {
        g = __uint_as_float(o.g);
        bt = bf16_to_f32((uint16_t)o.beta);
    } else {
        // An absent token keeps decay 1 (its other operands are all zero): the gate is
        // computed either way and masked, with no branch. A uniform branch here let the
        // compiler sink the tile loads below it, after the gate loads and their waits.
        const float sp = o.ds * softplus_fast(gate_value<GATE == kGateF16>(o.g) + o.dt);
        g = __uint_as_float(__float_as_uint(sp) & (0u - (uint32_t)o.present));
        bt = sigmoid_fast(gate_value<GATE == kGateF16>(o.beta));
    }
    const float eg = __expf(g);
    float ks = 1.f, qs = scale;
    if constexpr (GATE != kGateGiven) {
        // Optional L2 normalisation, also without a branch (the wave holds the whole head
        // vector, RPL values per lane).
        float kss = 0.f, qss = 0.f;
#pragma unroll
        for (int j = 0; j < Sh::RPL; ++j) {
            const float kv = __uint_as_float(j ? o.k & 0xFFFF0000u : o.k << 16);
            const float qv = __uint_as_float(j ? o.q & 0xFFFF0000u : o.q << 16);
            kss = fmaf(kv, kv, kss);
            qss = fmaf(qv, qv, qss);
        }
        const float kn = inv_norm(group_sum<64>(kss)), qn = inv_norm(group_sum<64>(qss));
        ks = norm ? kn : 1.f;
        qs = norm ? scale * qn : scale;
    }
#pragma unroll
    for (int j = 0; j < Sh::RPL; ++j) {
        const uint32_t kb = j ? o.k & 0xFFFF0000u : o.k << 16;
        const uint32_t qb = j ? o.q & 0xFFFF0000u : o.q << 16;
        *reinterpret_cast<f32x4 *>(ob + 4 * (lane * Sh::RPL + j)) =
            f32x4{eg * __expf(o.gk[j]), __uint_as_float(kb) * ks, __uint_as_float(qb) * qs, 0.f};
    }
    if constexpr (Sh::VPL == 2)
        *reinterpret_cast<float2 *>(ob + 4 * DK + 2 * lane) = make_float2(bf16_lo(o.v), bf16_hi(o.v));
    else
        ob[4 * DK + lane] = bf16_lo(o.v);
    return bt;
}

template <int DK, int TVW>
__device__ __forceinline__ void wave_load_state(const DecodeArgs &a, const Item &m,
                                                u32x4 (&raw)[WaveShape<DK, TVW>::RW], int cg,
                                                int rg) {
    using Sh = WaveShape<DK, TVW>;
    const auto rs = make_rsrc(a.pool + (m.state ? tile_base<DK, TVW>(a, m) : 0),
                              tile_range<DK, TVW>(a, m));
    // Per-lane part of the offset in a vector register, the per-row part (uniform) in the
    // instruction's scalar offset, so the loop keeps one offset register, not RW of them.
    const uint32_t lane_off = (uint32_t)((rg * a.Dv + cg * 8) * 2);
    const uint32_t row_step = (uint32_t)(Sh::RG * a.Dv * 2);
#pragma unroll
    for (int r = 0; r < Sh::RW; ++r)
        raw[r] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, r * row_step,
                                                       RGDR_STATE_LOAD_POLICY);
}

template <int DK, int TVW, int GATE, bool OPS_FIRST>
__global__ __launch_bounds__(64, RGDR_WAVE_MIN_WAVES) void decode_wave_kernel(
    const DecodeArgs a, const int32_t *__restrict__ lens, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nacc) {
    using Sh = WaveShape<DK, TVW>;
    constexpr int RW = Sh::RW, RG = Sh::RG, LPW = Sh::LPW;
    __shared__ f32x4 lds4[Sh::OPS / 4];
    float *ob = reinterpret_cast<float *>(lds4);
    const int lane = threadIdx.x;
    const int cg = lane % LPW, rg = lane / LPW;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const Item m = resolve(a, Index{lens, idx, nacc}, a.item0 + xcd_item(blockIdx.x, gridDim.x));
    // Load order. Large launches request the tile first, then the operands: staging the
    // operands then waits for the whole tile (the vector memory counter is in order), which
    // costs nothing because the reduction needs all of it anyway, and the tile's requests
    // reach the saturated memory queues sooner (22.9 against 23.4 us at B = 64, H_v = 32,
    // D = 128; 94.4 against 96.2 us at B = 256). Small launches, whose memory queues are
    // not full, request the operands first, so the gate and staging arithmetic runs while
    // the tile is in flight (B = 8: 6.5 against 7.4 us; B = 16: 7.8 against 9.1 us; one
    // sequence of 64 heads at D_k = 64, D_v = 512: 5.0 against 5.4 us). The scheduling fence
    // keeps the compiler from merging the two groups. The staging has no branch: the
    // compiler sinks loads whose results are used only after a branch below them.
    u32x4 W[RW];
    WaveOps<DK> ops;
    if constexpr (OPS_FIRST) {
        wave_load_ops<DK, TVW, GATE>(a, m, ops, lane);
        __builtin_amdgcn_sched_barrier(0);
        wave_load_state<DK, TVW>(a, m, W, cg, rg);
    } else {
        wave_load_state<DK, TVW>(a, m, W, cg, rg);
        wave_load_ops<DK, TVW, GATE>(a, m, ops, lane);
    }
    const float bt = wave_stage_ops<DK, TVW, GATE>(ops, ob, a.scale, a.norm_qk != 0, lane);

    // Step 1 (decay) fused with the partial sums of steps 2 and 4.
    float pk[8], pq[8];
    float kq = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) pk[c] = pq[c] = 0.f;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const f32x4 dkq = *reinterpret_cast<const f32x4 *>(ob + 4 * (rg + RG * r));
        const float d = dkq.x, kk = dkq.y, qq = dkq.z;
        kq = fmaf(kk, qq, kq);
        // (S_ij d_i) k_i summed over i, as S_ij (d_i k_i): the decay folds into the FMA.
        const float dk = d * kk, dq = d * qq;
        const uint32_t w[4] = {W[r].x, W[r].y, W[r].z, W[r].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float s0 = bf16_lo(w[j]), s1 = bf16_hi(w[j]);
            pk[2 * j] = fmaf(s0, dk, pk[2 * j]);
            pq[2 * j] = fmaf(s0, dq, pq[2 * j]);
            pk[2 * j + 1] = fmaf(s1, dk, pk[2 * j + 1]);
            pq[2 * j + 1] = fmaf(s1, dq, pq[2 * j + 1]);
        }
    }
    // Full sums over D_k: the row groups of this wave are LPW lanes apart.
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        pk[c] = colsum<LPW>(pk[c]);
        pq[c] = colsum<LPW>(pq[c]);
    }
    kq = colsum<LPW>(kq);
    const f32x4 *vv = reinterpret_cast<const f32x4 *>(ob + 4 * DK + cg * 8);
    const f32x4 v0 = vv[0], v1 = vv[1];
    const float V[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    // Step 3 (delta update) and step 4 (output with the updated state).
    float u[8], o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        u[c] = bt * (V[c] - pk[c]);
        o[c] = fmaf(kq, u[c], pq[c]);
    }
    {
        const size_t bh = (size_t)m.b * a.Hv + m.h;
        const auto rout = make_rsrc(a.out + bh * a.Dv, (uint32_t)(a.Dv * 2));
        u32x4 ov;
        ov.x = pack_bf16x2(o[0], o[1]);
        ov.y = pack_bf16x2(o[2], o[3]);
        ov.z = pack_bf16x2(o[4], o[5]);
        ov.w = pack_bf16x2(o[6], o[7]);
        __builtin_amdgcn_raw_buffer_store_b128(
            ov, rout, rg == 0 ? (uint32_t)((m.tile * TVW + cg * 8) * 2) : 0x7FFFFFF0u, 0, 0);
    }
    // The update widens the packed tile again (decay and k re-read from LDS) instead of
    // keeping the reduction's widened values alive; the empty asm marks the packed
    // registers as redefined so the compiler cannot reuse those values.
#pragma unroll
    for (int r = 0; r < RW; ++r) asm volatile("" : "+v"(W[r]));
    // Commit hold: no tile is written back before the launch's reads could all have
    // completed (a.hold, set by launch_wave). HBM streams reads and writes best in separate
    // phases, and waves whose tiles arrive early would otherwise start writing while most
    // reads are still in flight. The wait is bounded by the clock and by an iteration cap,
    // so it ends whatever other work shares the device; results never depend on it.
    if (a.hold > 0) {
        const uint64_t until = t0 + (uint64_t)a.hold;
        for (int i = 0; i < kHoldMaxPolls; ++i) {
            if (__builtin_amdgcn_s_memrealtime() >= until) break;
            __builtin_amdgcn_s_sleep(2);
        }
    }
    const auto rso = make_rsrc(a.pool_out + (m.state ? tile_base<DK, TVW>(a, m) : 0),
                               tile_range<DK, TVW>(a, m));
    const uint32_t lane_off = (uint32_t)((rg * a.Dv + cg * 8) * 2);
    const uint32_t row_step = (uint32_t)(RG * a.Dv * 2);
    if (m.n == 0) {  // nothing accepted: commit the incoming bytes
#pragma unroll
        for (int r = 0; r < RW; ++r)
            store16<RGDR_STATE_STORE_POLICY>(W[r], rso, lane_off + r * row_step);
    } else {
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const f32x4 dkq = *reinterpret_cast<const f32x4 *>(ob + 4 * (rg + RG * r));
            const uint32_t w[4] = {W[r].x, W[r].y, W[r].z, W[r].w};
            uint32_t nw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                nw[j] = pack_bf16x2(fmaf(dkq.y, u[2 * j], bf16_lo(w[j]) * dkq.x),
                                    fmaf(dkq.y, u[2 * j + 1], bf16_hi(w[j]) * dkq.x));
            store16<RGDR_STATE_STORE_POLICY>(u32x4{nw[0], nw[1], nw[2], nw[3]}, rso,
                                             lane_off + r * row_step);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Wave form for 1 < T <= 8 where the chunk form does not apply (D_v not a multiple of
// 128): one wave owns one (b, h, TV-column) tile over all D_k rows and
// keeps it in fp32 registers through the tokens (R rows x 8 columns per lane, 128 values at
// most); per token the D_k reduction finishes inside the wave, with no barrier and no LDS
// exchange. One item per wave; the operands of all of the item's tokens are staged once in
// the wave's LDS area.
//
// Scaled state. The tile is kept as S = diag(c) St, c_i the decay of row i not yet applied
// to St. Token t multiplies c by its decay d_t = exp(g_t) exp(gk_t), so step 1 costs
// nothing per element: steps 2 and 4 read St against (c k) and (c scale q), and step 3 adds
// (k / c) (x) u to St. That is three FMAs per element and token instead of four. The c of
// every row and token is formed once, at staging; where some row's c would leave
// [2^-64, 2^64] the token instead folds c d_t into St (one multiply per element) and
// restarts c at 1, so c, 1/c and St stay far from overflow and underflow. The commit
// multiplies St by the c of that token.
// ---------------------------------------------------------------------------------------

// Cross-lane reduction "transposed": the lanes LPR apart hold partial sums of the same 8
// columns over different rows. Each level exchanges half of a lane's values with its partner
// (v_permlane32_swap: lane ^ 32; v_permlane16_swap: lane ^ 16; a DPP rotate by 8 within 16
// lanes: lane ^ 8) and halves the number of values the lane carries, so in the end lane
// (cg, rg) holds complete sums of its own columns only: column rg of its group's 8 when
// LPR = 8, columns 2 rg and 2 rg + 1 when LPR = 16. Each sum is formed by one lane.
// 8 columns -> 4: out[c] is column c (lanes 0-31) or c + 4 (lanes 32-63), summed over lane ^ 32.
__device__ __forceinline__ void fold32(const float (&in)[8], float (&out)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float2 s = swap32(in[c], in[c + 4]);
        out[c] = s.x + s.y;
    }
}
// 4 -> 2: out[c] is column c (+4 as before) in even 16-lane rows, c + 2 in odd rows.
__device__ __forceinline__ void fold16(const float (&in)[4], float (&out)[2]) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const float2 s = swap16(in[c], in[c + 2]);
        out[c] = s.x + s.y;
    }
}
// 2 -> 1: column in[0] on lanes with bit 3 clear, in[1] on lanes with bit 3 set.
__device__ __forceinline__ float fold8(const float (&in)[2], bool b3) {
    const float x = b3 ? in[1] : in[0], y = b3 ? in[0] : in[1];
    return x + lane_xor8(y);
}
// The inverse: every lane of a column group gathers the 8 values of its group's columns.
__device__ __forceinline__ void spread8(float u, bool b3, float (&out)[2]) {
    const float w = lane_xor8(u);
    out[0] = b3 ? w : u;
    out[1] = b3 ? u : w;
}
__device__ __forceinline__ void spread16(const float (&in)[2], float (&out)[4]) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float2 s = swap16(in[k], in[k]);
        out[k] = s.x;
        out[k + 2] = s.y;
    }
}
__device__ __forceinline__ void spread32(const float (&in)[4], float (&out)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float2 s = swap32(in[j], in[j]);
        out[j] = s.x;
        out[j + 4] = s.y;
    }
}

// Second staging pass of the multi-token form: rewrite each row's (d, k, scale q) of every
// token as (c k, c scale q, k / c, fold multiplier), with c the running decay described
// above, and store per token the scalar k.(scale q) and whether the token folds. cc
// receives each row's c after token n - 1 (the commit), and cs (with SNAP) each row's c
// after every token, [t][D_k]. Lane l owns rows l and l + 64.
template <int DK, int TV, bool SNAP = false>
__device__ __forceinline__ void scale_ops(float *ob, float *cc, float *cs, int L, int n, int lane) {
    using Sh = TileShape<DK, TV, 64, kMaxT>;
    constexpr int RL = DK / 64;
    float c[RL];
#pragma unroll
    for (int j = 0; j < RL; ++j) c[j] = 1.f;
    for (int t = 0; t < L; ++t) {
        float *tb = ob + t * Sh::TOK;
        f32x4 e[RL];
        float cp[RL];
        bool out_of_range = false;
#pragma unroll
        for (int j = 0; j < RL; ++j) {
            e[j] = *reinterpret_cast<const f32x4 *>(tb + 4 * (lane + 64 * j));
            cp[j] = c[j] * e[j].x;
            out_of_range |= !(cp[j] >= 0x1p-64f && cp[j] <= 0x1p64f);
        }
        const bool fold = __ballot(out_of_range) != 0;  // wave-uniform
        float kqs = 0.f;
#pragma unroll
        for (int j = 0; j < RL; ++j) {
            const float r = fold ? cp[j] : 1.f;
            c[j] = fold ? 1.f : cp[j];
            kqs = fmaf(e[j].y, e[j].z, kqs);
            *reinterpret_cast<f32x4 *>(tb + 4 * (lane + 64 * j)) =
                f32x4{c[j] * e[j].y, c[j] * e[j].z, e[j].y * __builtin_amdgcn_rcpf(c[j]), r};
        }
        kqs = group_sum<64>(kqs);
        if (lane == 0) {
            tb[4 * DK + TV + 1] = kqs;
            tb[4 * DK + TV + 2] = fold ? 1.f : 0.f;
        }
        if (t + 1 == n) {
#pragma unroll
            for (int j = 0; j < RL; ++j) cc[lane + 64 * j] = c[j];
        }
        if constexpr (SNAP) {
#pragma unroll
            for (int j = 0; j < RL; ++j) cs[t * DK + lane + 64 * j] = c[j];
        }
    }
}

template <int DK, int TV, int GATE, bool SNAP = false>
__global__ __launch_bounds__(64, RGDR_WAVE_MIN_WAVES) void decode_wave_multi_kernel(
    const DecodeArgs a, const int32_t *__restrict__ lens, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nacc) {
    using Sh = TileShape<DK, TV, 64, kMaxT>;
    constexpr int LPR = Sh::LPR, RPP = Sh::RPP, R = Sh::R;
    static_assert(R * Sh::CPL <= 128, "fp32 tile per lane");
    static_assert(DK == 64 || DK == 128, "rows per lane in scale_ops");
    static_assert(LPR == 8 || LPR == 16, "transposed reduction");
    // per token: rows (4 floats) | v[TV] | beta, k.(scale q), fold flag, pad; then cc[DK];
    // with SNAP, each row's c after every token [kMaxT][DK]
    __shared__ f32x4 lds4[(Sh::OPS + DK + (SNAP ? kMaxT * DK : 0)) / 4];
    float *ob = reinterpret_cast<float *>(lds4);
    float *cc = ob + Sh::OPS;
    float *cs = cc + DK;
    const Index x{lens, idx, nacc};
    const int lane = threadIdx.x;
    const int cg = lane % LPR, rg = lane / LPR;
    const bool b3 = (lane >> 3) & 1;
    const Item m = resolve(a, x, a.item0 + xcd_item(blockIdx.x, gridDim.x));

    Ops<DK, TV, 64, kMaxT> o;
    load_ops<DK, TV, 64, kMaxT, GATE>(a, m, o, lane);
    u32x4 raw[R];
    load_state<DK, TV, 64>(a, m, raw, rg, cg);
    stage_ops<DK, TV, 64, kMaxT, GATE>(o, ob, a.scale, a.norm_qk != 0, lane);
    scale_ops<DK, TV, SNAP>(ob, cc, cs, m.L, m.n, lane);

    const auto rso = make_rsrc(a.pool_out + (m.state ? tile_base<DK, TV>(a, m) : 0),
                               tile_range<DK, TV>(a, m));
    const uint32_t lane_off = (uint32_t)((rg * a.Dv + cg * 8) * 2);
    const uint32_t row_step = (uint32_t)(RPP * a.Dv * 2);
    if (m.n == 0) {  // nothing accepted: commit the incoming bytes
#pragma unroll
        for (int r = 0; r < R; ++r)
            store16<RGDR_STATE_STORE_POLICY>(raw[r], rso, lane_off + r * row_step);
    }
    float S[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t w[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            S[r][2 * j] = bf16_lo(w[j]);
            S[r][2 * j + 1] = bf16_hi(w[j]);
        }
    }
    const size_t bh = (size_t)m.b * a.Hv + m.h;
    const auto rout = make_rsrc(a.out + bh * a.T * a.Dv, (uint32_t)(a.T * a.Dv * 2));
    // the lane's own output column(s) within the tile
    constexpr int OWN = LPR == 8 ? 1 : 2;
    const int col = cg * 8 + rg * OWN;
    const uint32_t ocol = (uint32_t)((m.tile * TV + col) * 2);
    for (int t = 0; t < m.L; ++t) {
        const float *tb = ob + t * Sh::TOK;
        const float bt = tb[4 * DK + TV], kq = tb[4 * DK + TV + 1];
        if (__builtin_amdgcn_readfirstlane(__float_as_int(tb[4 * DK + TV + 2])) != 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float f = tb[4 * (rg + RPP * r) + 3];
#pragma unroll
                for (int c = 0; c < 8; ++c) S[r][c] *= f;
            }
        }
        // Steps 2 and 4 (step 1 is in the multipliers): partial sums over the lane's rows.
        float P[8], Q[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) P[c] = Q[c] = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const f32x4 mul = *reinterpret_cast<const f32x4 *>(tb + 4 * (rg + RPP * r));
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                P[c] = fmaf(S[r][c], mul.x, P[c]);
                Q[c] = fmaf(S[r][c], mul.y, Q[c]);
            }
        }
        float P4[4], Q4[4], P2[2], Q2[2];
        fold32(P, P4);
        fold32(Q, Q4);
        fold16(P4, P2);
        fold16(Q4, Q2);
        // Step 3's u and step 4's output for the lane's own column(s), then u for all 8.
        float U[8];
        if constexpr (LPR == 8) {
            const float p = fold8(P2, b3), q = fold8(Q2, b3);
            const float u = bt * (tb[4 * DK + col] - p);
            const float ov = fmaf(kq, u, q);
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(ov), rout,
                                                  (uint32_t)(t * a.Dv * 2) + ocol, 0, 0);
            float U2[2], U4[4];
            spread8(u, b3, U2);
            spread16(U2, U4);
            spread32(U4, U);
        } else {
            float U2[2], U4[4], ov[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                U2[k] = bt * (tb[4 * DK + col + k] - P2[k]);
                ov[k] = fmaf(kq, U2[k], Q2[k]);
            }
            __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(ov[0], ov[1]), rout,
                                                  (uint32_t)(t * a.Dv * 2) + ocol, 0, 0);
            spread16(U2, U4);
            spread32(U4, U);
        }
        // Step 3: St += (k / c) (x) u.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float kc = tb[4 * (rg + RPP * r) + 2];
#pragma unroll
            for (int c = 0; c < 8; ++c) S[r][c] = fmaf(kc, U[c], S[r][c]);
        }
        if constexpr (SNAP) {  // the state after token t: c St, as the commit below
            const size_t sb = (((size_t)m.b * a.T + t) * a.Hv + m.h) * DK * a.Dv +
                              (size_t)m.tile * TV;
            const auto rsn = make_rsrc(a.snap + sb, (uint32_t)(DK * a.Dv - m.tile * TV) * 2);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float cr = cs[t * DK + rg + RPP * r];
                store16<RGDR_STATE_STORE_POLICY>(
                    u32x4{pack_bf16x2(S[r][0] * cr, S[r][1] * cr),
                          pack_bf16x2(S[r][2] * cr, S[r][3] * cr),
                          pack_bf16x2(S[r][4] * cr, S[r][5] * cr),
                          pack_bf16x2(S[r][6] * cr, S[r][7] * cr)},
                    rsn, lane_off + r * row_step);
            }
        }
        if (t + 1 == m.n) {  // the accepted prefix ends here: commit c St
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float cr = cc[rg + RPP * r];
                store16<RGDR_STATE_STORE_POLICY>(
                    u32x4{pack_bf16x2(S[r][0] * cr, S[r][1] * cr),
                          pack_bf16x2(S[r][2] * cr, S[r][3] * cr),
                          pack_bf16x2(S[r][4] * cr, S[r][5] * cr),
                          pack_bf16x2(S[r][6] * cr, S[r][7] * cr)},
                    rso, lane_off + r * row_step);
            }
        }
    }
    for (int t = m.L; t < a.T; ++t) {  // padded (or skipped) tokens: +0.0 rows
        if constexpr (LPR == 8)
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, rout, (uint32_t)(t * a.Dv * 2) + ocol, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(0u, rout, (uint32_t)(t * a.Dv * 2) + ocol, 0, 0);
    }
}

// ---------------------------------------------------------------------------------------
// Chunk form for 1 < T <= 8 at D_k = 64 or 128 with 128-column tiles: the item's L tokens are
// evaluated together, on the matrix cores where the work is a dense contraction.
//
// With d_t the row decays of token t, c_t = d_0 ... d_t and g(t,s) = d_{s+1} ... d_t
// (g(t,t) = 1; every factor lies in [0, 1] for decays, so nothing here can overflow), the
// recurrence unrolls exactly to
//   p_t = S0^T (c_t k_t)        + sum_{s<t}  M[t][s] u_s,  M[t][s] = sum_i g(t,s)_i k_s,i k_t,i
//   o_t = S0^T (c_t scale q_t)  + sum_{s<=t} N[t][s] u_s,  N[t][s] = sum_i g(t,s)_i k_s,i scale q_t,i
//   u_t = beta_t (v_t - p_t)
//   S_n = diag(c_{n-1}) S0 + sum_{s<n} (g(n-1,s) k_s) (x) u_s        (the committed state)
// The two sums over D_k x D_v x L (S0^T [c k | c scale q], and the rank-n update) are bf16
// 16x16x32 MFMAs with fp32 accumulation: S0 is bf16 already, and every fp32 operand is split
// into a bf16 high part and a bf16 remainder, so the products keep about 16 bits of each
// operand. The rest (decay products, the 8 x 8 matrices M and N, the triangular solve for u,
// column by column, and the row scaling diag(c) S0 that starts each commit accumulator) is
// fp32 VALU.
//
// Two waves per item. Wave w owns tile columns 64 w .. 64 w + 63 over all D_k rows, so
// each wave's contraction, solve and update are complete for its columns; only the per-row
// preparation (thread r: row r; at D_k = 64 wave 0 alone) is shared, through LDS, and two
// workgroup barriers suffice (operands staged; rows prepared). At D_k = 128 four items fit
// one compute unit, two waves per SIMD.
//
// Lane layout. Lane l = (kg, n16) = (l / 16, l % 16) of wave w loads rows 16 rb + 4 kg + i
// (rb < D_k / 16, i < 4), columns 64 w + 4 n16 .. + 3: 16 lanes cover the wave's 128 bytes of a
// row. For the contraction the tile's row index is the k index (the 8 k slots of lane group
// kg hold its rows 4 kg + i of two row blocks) and column 64 w + 4 n + c is element n of
// column set c. In the commit the accumulator of block (rb, c) holds exactly the lane's own
// elements of rows 16 rb + 4 kg + i, column 64 w + 4 n16 + c: the lane scales its own loaded
// values into it, and the update lands in the layout the commit stores.
//
// SNAP (the snapshot entries): the state after token t is the same expression with n - 1
// replaced by t, S_t = diag(c_t) S0 + sum_{s<=t} (g(t,s) k_s) (x) u_s, so after the solve the
// commit's products are taken once per t < L, with each row's weights for t, and stored to
// snapshot t (and, for t = n - 1, to the pool).
// ---------------------------------------------------------------------------------------

// The chunk form serves calls with T >= RGDR_CHUNK_MIN_T. Its time hardly depends on the
// tokens per item; the per-token form's grows with the longest item, and is no lower even at
// 2 tokens.
#ifndef RGDR_CHUNK_FORM
#define RGDR_CHUNK_FORM 1
#endif
#ifndef RGDR_CHUNK_MIN_T
#define RGDR_CHUNK_MIN_T 2
#endif
// The chunk form at D_k = 64 too (0: those calls take the per-token form), from
// RGDR_CHUNK_DK64_MIN_T tokens. At D_k = 64 a chunk-form item holds half the state bytes
// for the same fixed work, and its LDS fits five items per compute unit, so large calls
// need more rounds of items than the per-token form needs of waves. Measured, all lengths T
// (chunk against per-token): B = 64, H = 32, D_v = 128: T = 2 17.9 against 13.0 us, T = 3
// 18.3 against 15.0, T = 4 19.3 against 16.8, T = 5 18.7 against 18.7; B = 16, H = 64,
// D_v = 512: T = 2 29.8 against 29.3, T = 3 29.8 against 31.4, and at T = 8 (varlen)
// 30.8 against 37.8.
#ifndef RGDR_CHUNK_DK64
#define RGDR_CHUNK_DK64 1
#endif
#ifndef RGDR_CHUNK_DK64_MIN_T
#define RGDR_CHUNK_DK64_MIN_T 5
#endif
// The chunk form for D_v an odd multiple of 64 too, with a last tile of 64 columns (0: those
// calls take the per-token form). The half tile leaves one of its two waves idle. Measured,
// H = 32, D_k = 128, all lengths T (chunk against per-token): D_v = 192, B = 32: T = 2 24.6
// against 25.8 us, T = 3 24.2 against 27.3, T = 8 25.7 against 39.1; D_v = 320, T = 3 35.8
// against 39.5. At D_v = 64 every tile is half: B = 16 gains from T = 3 (8.7 against
// 9.1 us), but B = 64 needs two rounds of items and loses at T = 4 (21.2 against 19.3 us),
// ties near T = 5 and gains at T = 6 (21.4 against 23.2). D_v = 64 therefore takes the chunk
// form from RGDR_CHUNK_DV64_MIN_T tokens.
#ifndef RGDR_CHUNK_HALF_TILE
#define RGDR_CHUNK_HALF_TILE 1
#endif
#ifndef RGDR_CHUNK_DV64_MIN_T
#define RGDR_CHUNK_DV64_MIN_T 5
#endif
// Where the chunk form issues its tile loads: RGDR_CHUNK_PRE row blocks with the operand
// loads, RGDR_CHUNK_POST more once the operands are staged, the rest one block per token
// step of the per-row preparation.
#ifndef RGDR_CHUNK_PRE
#define RGDR_CHUNK_PRE 3
#endif
#ifndef RGDR_CHUNK_POST
#define RGDR_CHUNK_POST 1
#endif


template <int DK, int GATE, bool SNAP = false>
__global__ __launch_bounds__(128, 2) void decode_chunk_kernel(
    const DecodeArgs a, const int32_t *__restrict__ lens, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nacc) {
    static_assert(DK == 64 || DK == 128, "chunk form: D_k = 64 or 128");
    constexpr int TV = 128, NT = 128;
    constexpr int NRB = DK / 16, NPB = DK / 32;  // row blocks of the tile, and their pairs
    // LDS: staged operands (chunk_stage_ops) | XT hi, lo [16][XS] | KA hi, lo [D_k][8] |
    // UT [wave][hi, lo] [4 column sets][16][8] | c_{n-1} per row | G partials [wave][64] |
    // M and N [wave][8][8]. Y^T [128][16] fp32 (one tile column per 80-byte row)
    // takes the d, k and q planes of the staged operands once both waves have prepared their
    // rows. The row stride of XT is padded (XS = D_k + 4) so the fragment reads of the 16
    // lanes of a lane group fall in different LDS banks; UT is ordered by column set for the
    // same reason. At D_k = 64 only wave 0 has rows to prepare.
    constexpr int XS = DK + 4;
    constexpr int VB = chunk_vbase<DK>();  // v plane, then beta, in the staged operands
    constexpr int OFF_XT = chunk_ops<DK>() * 4;
    constexpr int OFF_KA = OFF_XT + 2 * 16 * XS * 2;
    constexpr int OFF_UT = OFF_KA + 2 * DK * 8 * 2;
    constexpr int OFF_CL = OFF_UT + 2 * 2 * 64 * 8 * 2;
    constexpr int OFF_GP = OFF_CL + DK * 4;
    constexpr int OFF_GS = OFF_GP + 2 * 64 * 4;
    constexpr int BYTES = OFF_GS + 2 * 2 * 64 * 4;
    static_assert(BYTES % 16 == 0 && BYTES <= 40960, "LDS carve: four items per compute unit");
    constexpr int YS = kChunkYS;
    static_assert(128 * YS <= VB && (YS * 4) % 16 == 0, "Y^T fits the d, k, q planes");
    static_assert(chunk_ops<DK>() % 4 == 0 && (2 * 16 * XS * 2) % 16 == 0, "16-byte aligned carve");
    __shared__ f32x4 lds4[BYTES / 16];
    char *lb = reinterpret_cast<char *>(lds4);
    float *ob = reinterpret_cast<float *>(lb);
    uint16_t *xt_hi = reinterpret_cast<uint16_t *>(lb + OFF_XT), *xt_lo = xt_hi + 16 * XS;
    uint16_t *ka_hi = reinterpret_cast<uint16_t *>(lb + OFF_KA), *ka_lo = ka_hi + DK * 8;
    float *crow = reinterpret_cast<float *>(lb + OFF_CL);
    float *gpart = reinterpret_cast<float *>(lb + OFF_GP);

    const Index x{lens, idx, nacc};
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n16 = lane & 15, kg = lane >> 4;
    uint16_t *ut_hi = reinterpret_cast<uint16_t *>(lb + OFF_UT) + w * 2 * 64 * 8, *ut_lo = ut_hi + 64 * 8;
    float *gsM = reinterpret_cast<float *>(lb + OFF_GS) + w * 2 * 64, *gsN = gsM + 64;
    const Item m = resolve(a, x, a.item0 + xcd_item(blockIdx.x, gridDim.x));
    const int L = m.L, n = m.n;
    auto ycol = [&](int j) { return ob + j * YS; };

    // The operands first, with a few row blocks of the tile (PRE); more once the operands
    // are staged (POST); the rest one block per token step of the per-row preparation. Issued
    // all at once, the tile loads would block the wave for microseconds (the memory queues
    // are full) before it could stage or prepare anything; issued after the operands alone,
    // the memory system would idle while they arrive.
    constexpr int PRE = RGDR_CHUNK_PRE < NRB ? RGDR_CHUNK_PRE : NRB;
    constexpr int POST = RGDR_CHUNK_POST < NRB - PRE ? RGDR_CHUNK_POST : NRB - PRE;
    static_assert(PRE >= 0 && POST >= 0 && PRE + POST <= NRB, "tile load placement");
    // Row blocks left for the preparation are issued by every thread's loop, so each wave
    // must prepare rows then: true at D_k = 128; at D_k = 64 none are left.
    static_assert(DK == 128 || PRE + POST == NRB, "interleaved loads need rows in both waves");
    // A last tile of 64 columns (D_v an odd multiple of 64) leaves wave 1 without columns:
    // its tile, output and state accesses get empty ranges (its columns would alias the
    // next row's), and it computes on zeros that nothing reads.
    // (w is the same in every lane of a wave; readfirstlane tells the compiler so, which
    // keeps the buffer descriptors built from it in scalar registers.)
    const bool cols = m.tile * TV + 64 * __builtin_amdgcn_readfirstlane(w) < a.Dv;
    const uint32_t trange = cols ? tile_range<DK, TV>(a, m) : 0u;
    const auto rs = make_rsrc(a.pool + (m.state ? tile_base<DK, TV>(a, m) : 0), trange);
    const uint32_t lane_off = (uint32_t)((4 * kg * a.Dv + 64 * w + 4 * n16) * 2);
    u32x2 raw[NRB][4];
    auto load_rb = [&](int rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            raw[rb][i] = __builtin_amdgcn_raw_buffer_load_b64(
                rs, lane_off, (uint32_t)((16 * rb + i) * a.Dv * 2), RGDR_STATE_LOAD_POLICY);
    };
    Ops<DK, TV, NT, kMaxT> o;
    load_ops<DK, TV, NT, kMaxT, GATE>(a, m, o, tid);
#pragma unroll
    for (int rb = 0; rb < PRE; ++rb) load_rb(rb);
    __builtin_amdgcn_sched_barrier(0);
    chunk_stage_ops<DK, GATE>(o, ob, a.scale, a.norm_qk != 0, L, tid);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rb = PRE; rb < PRE + POST; ++rb) load_rb(rb);
    lds_barrier();

    // Per-row preparation: thread r owns row r (uniform per wave: at D_k = 64 wave 1 has none).
    float gp[64];  // partial G: [t][s] (s <= t) holds N[t][s], [s][t] (s < t) holds M[t][s]
#pragma unroll
    for (int e = 0; e < 64; ++e) gp[e] = 0.f;
    const bool has_rows = 64 * w < DK;
    float dkeep[8], kkeep[8];  // with SNAP, this thread's row: decay and k per token
    if (has_rows) {
        const int row = tid;
        float d[8], k[8], q[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            d[t] = ob[t * DK + row];  // padded tokens were staged neutral
            k[t] = ob[8 * DK + t * DK + row];
            q[t] = ob[16 * DK + t * DK + row];
        }
        if constexpr (SNAP) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                dkeep[t] = d[t];
                kkeep[t] = k[t];
            }
        }
        float c = 1.f, cnv = 1.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (PRE + POST + t < NRB) {  // the remaining tile loads, one row block per step
                __builtin_amdgcn_sched_barrier(0);
                load_rb(PRE + POST + t);
                __builtin_amdgcn_sched_barrier(0);
            }
            c *= d[t];
            uint16_t hk, lk, hq, lq;
            split_bf16(c * k[t], hk, lk);
            split_bf16(c * q[t], hq, lq);
            xt_hi[t * XS + row] = hk;
            xt_lo[t * XS + row] = lk;
            xt_hi[(8 + t) * XS + row] = hq;
            xt_lo[(8 + t) * XS + row] = lq;
            if (t + 1 == n) cnv = c;
        }
        crow[row] = cnv;  // this row's entry of diag(c_{n-1})
        float ka[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            float wv = k[s];  // g(s,s) k_s
            ka[s] = (s + 1 == n) ? wv : 0.f;
            gp[s * 8 + s] = wv * q[s];
#pragma unroll
            for (int t = s + 1; t < 8; ++t) {
                wv *= d[t];  // g(t,s) k_s
                gp[s * 8 + t] = wv * k[t];
                gp[t * 8 + s] = wv * q[t];
                if (t + 1 == n) ka[s] = wv;
            }
        }
        uint16_t kh[8], kl[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) split_bf16(ka[s], kh[s], kl[s]);
        *reinterpret_cast<u32x4 *>(ka_hi + row * 8) =
            u32x4{kh[0] | ((uint32_t)kh[1] << 16), kh[2] | ((uint32_t)kh[3] << 16),
                  kh[4] | ((uint32_t)kh[5] << 16), kh[6] | ((uint32_t)kh[7] << 16)};
        *reinterpret_cast<u32x4 *>(ka_lo + row * 8) =
            u32x4{kl[0] | ((uint32_t)kl[1] << 16), kl[2] | ((uint32_t)kl[3] << 16),
                  kl[4] | ((uint32_t)kl[5] << 16), kl[6] | ((uint32_t)kl[7] << 16)};
    }
    // G over this wave's 64 rows: lane e holds entry e.
    gpart[64 * w + lane] = has_rows ? wave_sum64_transposed(gp, lane) : 0.f;
    lds_barrier();
    {
        // Entry e = 8 a + b of G, summed over the two halves of the rows, into this wave's
        // tables: M[t][s] (s < t) and N[t][s] (s <= t), rows read as broadcast vectors.
        const float g_e = gpart[lane] + gpart[64 + lane];
        const int ea = lane >> 3, eb = lane & 7;
        if (ea < eb)
            gsM[eb * 8 + ea] = g_e;
        else
            gsN[ea * 8 + eb] = g_e;
    }
    lds_phase();

    // Y = [c k | c scale q]^T S0 (16 x 64, this wave's columns): column set c, accumulated
    // over row-block pairs; the k slots of lane group kg are rows 4 kg .. 4 kg + 3 of block
    // 2p, then of block 2p+1.
    auto frag8 = [](const s16x4 f0, const s16x4 f1) {
        const uint2 x = __builtin_bit_cast(uint2, f0), y = __builtin_bit_cast(uint2, f1);
        return __builtin_bit_cast(bf16x8, u32x4{x.x, x.y, y.x, y.y});
    };
    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
        const int r0 = 32 * pb + 4 * kg;
        const bf16x8 ah = lds_pair8(xt_hi + n16 * XS + r0, xt_hi + n16 * XS + r0 + 16);
        const bf16x8 al = lds_pair8(xt_lo + n16 * XS + r0, xt_lo + n16 * XS + r0 + 16);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8 bf = frag8(column_frag(raw[2 * pb], c), column_frag(raw[2 * pb + 1], c));
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bf, acc[c], 0, 0, 0);
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bf, acc[c], 0, 0, 0);
        }
    }
    // Y to LDS, transposed: accumulator c holds rows 4 kg .. 4 kg + 3 of column
    // 64 w + 4 n16 + c.
    lds_phase();
#pragma unroll
    for (int c = 0; c < 4; ++c)
        *reinterpret_cast<f32x4 *>(ycol(64 * w + 4 * n16 + c) + 4 * kg) = acc[c];

    lds_phase();
    // Triangular solve, column 64 w + lane; outputs; u of the accepted prefix.
    const int col = 64 * w + lane;
    const size_t bh = (size_t)m.b * a.Hv + m.h;
    const auto rout = make_rsrc(a.out + bh * a.T * a.Dv, cols ? (uint32_t)(a.T * a.Dv * 2) : 0u);
    const uint32_t ocol = (uint32_t)((m.tile * TV + col) * 2);
    float yc[16];  // this column of Y: [c k]^T S0 for t < 8, then [c scale q]^T S0
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
        const f32x4 e = *reinterpret_cast<const f32x4 *>(ycol(col) + 4 * v4);
        yc[4 * v4] = e.x;
        yc[4 * v4 + 1] = e.y;
        yc[4 * v4 + 2] = e.z;
        yc[4 * v4 + 3] = e.w;
    }
    // Straight-line over all 8 token slots (no branch on L, so the LDS reads can be issued
    // together): every staged value of a padded token is finite (its loads returned zeros),
    // and its u and output are masked to 0.
    float u[8];
    uint16_t o16[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float v = ob[VB + t * TV + col];
        const float bt = ob[VB + 8 * TV + t];
        float p = yc[t];
#pragma unroll
        for (int s2 = 0; s2 < t; ++s2) p = fmaf(gsM[t * 8 + s2], u[s2], p);
        u[t] = t < L ? bt * (v - p) : 0.f;
        float ov = yc[8 + t];
#pragma unroll
        for (int s2 = 0; s2 <= t; ++s2) ov = fmaf(gsN[t * 8 + s2], u[s2], ov);
        o16[t] = t < L ? f32_to_bf16(ov) : (uint16_t)0;  // padded (or skipped) tokens: +0.0
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
        if (t < a.T)
            __builtin_amdgcn_raw_buffer_store_b16(o16[t], rout, (uint32_t)(t * a.Dv * 2) + ocol, 0, 0);
    {
        uint16_t h[8], l[8];
#pragma unroll
        // (with SNAP every token's u: each state's k weights are zero past its last token)
        for (int s2 = 0; s2 < 8; ++s2) split_bf16(SNAP || s2 < n ? u[s2] : 0.f, h[s2], l[s2]);
        // local column j = 4 n + c goes to UT position c * 16 + n
        const int p = (lane & 3) * 16 + (lane >> 2);
        *reinterpret_cast<u32x4 *>(ut_hi + p * 8) =
            u32x4{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                  h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
        *reinterpret_cast<u32x4 *>(ut_lo + p * 8) =
            u32x4{l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16),
                  l[4] | ((uint32_t)l[5] << 16), l[6] | ((uint32_t)l[7] << 16)};
    }

    lds_phase();
    // Commit.
    const auto rso = make_rsrc(a.pool_out + (m.state ? tile_base<DK, TV>(a, m) : 0), trange);
    if (n == 0) {  // nothing accepted: the incoming bytes
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                store8<RGDR_STATE_STORE_POLICY>(raw[rb][i], rso,
                                                lane_off + (uint32_t)((16 * rb + i) * a.Dv * 2));
        if constexpr (!SNAP) return;
    }
    // S_n = diag(c_{n-1}) S0 + [g k]^T U, block by block. The row scaling of the bf16 tile is
    // an fp32 multiply on the VALU and gives each accumulator its initial value; the rank-n
    // update is then one 16x16x32 product per block: lane group kg carries A's tokens 0..7 of
    // its high part (kg even) or remainder (kg odd), against U's high part (kg < 2) or
    // remainder (kg >= 2), so the four products of the split parts are all taken at once.
    // Each accumulator sees one matrix-core instruction shape only.
    bf16x8 bu[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        bu[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                               (kg >= 2 ? ut_lo : ut_hi) + (c * 16 + n16) * 8));
    const uint16_t *ka_lane = ((kg & 1) ? ka_lo : ka_hi) + n16 * 8;
    auto commit = [&](const __amdgpu_buffer_rsrc_t &dst, const __amdgpu_buffer_rsrc_t &dst2,
                      bool both) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const f32x4 cr = *reinterpret_cast<const f32x4 *>(crow + 16 * rb + 4 * kg);
            const bf16x8 ak = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(ka_lane + 16 * rb * 8));
            f32x4 D[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                D[0][i] = cr[i] * bf16_lo(raw[rb][i].x);
                D[1][i] = cr[i] * bf16_hi(raw[rb][i].x);
                D[2][i] = cr[i] * bf16_lo(raw[rb][i].y);
                D[3][i] = cr[i] * bf16_hi(raw[rb][i].y);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
                D[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bu[c], D[c], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x2 pk{pack_bf16x2(D[0][i], D[1][i]), pack_bf16x2(D[2][i], D[3][i])};
                const uint32_t off = lane_off + (uint32_t)((16 * rb + i) * a.Dv * 2);
                store8<RGDR_STATE_STORE_POLICY>(pk, dst, off);
                if (both) store8<RGDR_STATE_STORE_POLICY>(pk, dst2, off);
            }
        }
    };
    if constexpr (!SNAP) {
        commit(rso, rso, false);
    } else {
        // The state after every token t < L, in token order: S_t = diag(c_t) S0 +
        // [g(t, .) k]^T U, the commit's products with each row's weights for t (zero past t).
        // The one for t = n - 1 is also the commit, stored to the pool from the same registers.
        const uint32_t srange = cols ? (uint32_t)(DK * a.Dv - m.tile * TV) * 2 : 0u;
        float c = 1.f;
        for (int t = 0; t < L; ++t) {  // uniform: L is the item's
            if (has_rows) {
                const int row = tid;
                float kt[8];
                float wv = 1.f;  // g(t, s) as s runs down from t
#pragma unroll
                for (int s2 = 7; s2 >= 0; --s2) {
                    kt[s2] = s2 <= t ? wv * kkeep[s2] : 0.f;
                    if (s2 <= t) wv *= dkeep[s2];
                }
                c *= dkeep[t];
                uint16_t kh[8], kl[8];
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2) split_bf16(kt[s2], kh[s2], kl[s2]);
                *reinterpret_cast<u32x4 *>(ka_hi + row * 8) =
                    u32x4{kh[0] | ((uint32_t)kh[1] << 16), kh[2] | ((uint32_t)kh[3] << 16),
                          kh[4] | ((uint32_t)kh[5] << 16), kh[6] | ((uint32_t)kh[7] << 16)};
                *reinterpret_cast<u32x4 *>(ka_lo + row * 8) =
                    u32x4{kl[0] | ((uint32_t)kl[1] << 16), kl[2] | ((uint32_t)kl[3] << 16),
                          kl[4] | ((uint32_t)kl[5] << 16), kl[6] | ((uint32_t)kl[7] << 16)};
                crow[row] = c;
            }
            lds_barrier();
            const size_t sb = (((size_t)m.b * a.T + t) * a.Hv + m.h) * DK * a.Dv +
                              (size_t)m.tile * TV;
            commit(make_rsrc(a.snap + sb, srange), rso, t + 1 == n);
            lds_barrier();  // every wave has read this token's weights
        }
    }
}

// Waves of decode_wave_kernel<DK, TVW, GATE> the current device holds at once (compute units
// times waves per compute unit), queried once per device; 0 if the query fails.
template <int DK, int TVW, int GATE>
static int resident_waves() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 0;
    // Both issue orders are launched (by the launch's size); a launch must fit one round of
    // either, so the smaller of the two occupancies counts.
    int per_cu_ops = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, decode_wave_kernel<DK, TVW, GATE, false>, 64, WaveShape<DK, TVW>::LDS_PAD) !=
            hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu_ops, decode_wave_kernel<DK, TVW, GATE, true>, 64,
            WaveShape<DK, TVW>::LDS_PAD) != hipSuccess)
        per_cu = 1;
    per_cu = per_cu_ops < per_cu ? per_cu_ops : per_cu;
    if (per_cu < 1) per_cu = 1;
    n = cus * per_cu;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Ticks of the device's constant wall clock per microsecond (100 on this part), queried once
// per device; 0 if the query fails (then no commit hold).
static int wall_ticks_per_us() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        khz < 1000)
        return 0;
    n = khz / 1000;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// The read rate the commit hold assumes, in GB/s: the environment variable
// RGDR_HOLD_READ_GBPS when it holds a number (0 turns the hold off), else the built-in
// RGDR_HOLD_READ_GBPS. Read once, at the first single-token call of the process.
static double hold_read_gbps_env() {
    const char *e = std::getenv("RGDR_HOLD_READ_GBPS");
    if (e && *e) {
        char *end = nullptr;
        const double v = std::strtod(e, &end);
        if (end != e && v >= 0.0) return v;
    }
    return RGDR_HOLD_READ_GBPS;
}
static double hold_read_gbps() {
    static const double gbps = hold_read_gbps_env();  // thread-safe one-time initialisation
    return gbps;
}

// T = 1: one wave per item. A call with more items than resident waves becomes launches of
// the resident grid, one after another on the stream. Each launch requests all of its tiles
// before its commits start, which streams faster than waves that walk several items and
// mix one item's commit with the next one's reads (71% against 63% of 8 TB/s at B = 256,
// H_v = 32, D = 128); launches of a smaller grid pay the ramp and drain more often.
template <int DK, int TVW, int GATE>
static hipError_t launch_wave(const DecodeArgs &a, const int32_t *lens, const int32_t *idx,
                              const int32_t *nacc, hipStream_t stream) {
    constexpr int pad = WaveShape<DK, TVW>::LDS_PAD;
    const int chunk = resident_waves<DK, TVW, GATE>();
    if (chunk <= 0) return hipErrorInvalidDevice;
    const int ticks_per_us = wall_ticks_per_us();
    const double gbps = hold_read_gbps();
    DecodeArgs c = a;
    for (int first = 0; first < a.n_items; first += chunk) {
        c.item0 = first;
        c.n_items = a.n_items - first < chunk ? a.n_items : first + chunk;
        // The launch's tile bytes at the assumed read rate, in clock ticks (bytes / (GB/s)
        // is in nanoseconds).
        const double read_ns =
            gbps > 0.0 ? (double)(c.n_items - first) * DK * TVW * 2 / gbps : 0.0;
        const double ticks = read_ns * 1e-3 * ticks_per_us;
        c.hold = ticks < 1e9 ? (int)ticks : 1000000000;
        const double tile_bytes = (double)(c.n_items - first) * DK * TVW * 2;
        if (tile_bytes <= kOpsFirstBytes)
            hipLaunchKernelGGL((decode_wave_kernel<DK, TVW, GATE, true>), dim3(c.n_items - first),
                               dim3(64), pad, stream, c, lens, idx, nacc);
        else
            hipLaunchKernelGGL((decode_wave_kernel<DK, TVW, GATE, false>), dim3(c.n_items - first),
                               dim3(64), pad, stream, c, lens, idx, nacc);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// 1 < T <= 8 with D_v not a multiple of 128: one wave per item, all items in one launch (the
// hardware starts waves as slots free up).
template <int DK, int TV, int GATE>
static hipError_t launch_wave_multi(const DecodeArgs &a, const int32_t *lens,
                                    const int32_t *idx, const int32_t *nacc,
                                    hipStream_t stream) {
    if (a.snap) {  // per-token states (the snapshot entries)
        hipLaunchKernelGGL((decode_wave_multi_kernel<DK, TV, GATE, true>), dim3(a.n_items),
                           dim3(64), 0, stream, a, lens, idx, nacc);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((decode_wave_multi_kernel<DK, TV, GATE, false>), dim3(a.n_items),
                       dim3(64), 0, stream, a, lens, idx, nacc);
    return hipGetLastError();
}

// 2 <= T <= 8 with D_v a multiple of 128: one workgroup of two waves per item, all items in
// one launch.
template <int DK, int GATE>
static hipError_t launch_chunk(const DecodeArgs &a, const int32_t *lens, const int32_t *idx,
                               const int32_t *nacc, hipStream_t stream) {
    if (a.snap) {  // per-token states (the snapshot entries)
        hipLaunchKernelGGL((decode_chunk_kernel<DK, GATE, true>), dim3(a.n_items), dim3(128), 0,
                           stream, a, lens, idx, nacc);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((decode_chunk_kernel<DK, GATE>), dim3(a.n_items), dim3(128), 0, stream, a,
                       lens, idx, nacc);
    return hipGetLastError();
}

enum Form { kFormWave = 0, kFormWaveMulti = 1, kFormChunk = 2 };

template <int GATE>
static hipError_t dispatch(const DecodeArgs &a, int D_k, int tile_v, Form form,
                           const int32_t *L, const int32_t *I, const int32_t *N,
                           hipStream_t stream) {
    if (form == kFormChunk)
        return D_k == 128 ? launch_chunk<128, GATE>(a, L, I, N, stream)
                          : launch_chunk<64, GATE>(a, L, I, N, stream);
    if (form == kFormWaveMulti) {
        if (D_k == 128) return launch_wave_multi<128, 64, GATE>(a, L, I, N, stream);
        return tile_v == 128 ? launch_wave_multi<64, 128, GATE>(a, L, I, N, stream)
                             : launch_wave_multi<64, 64, GATE>(a, L, I, N, stream);
    }
    if (tile_v == 128)
        return D_k == 128 ? launch_wave<128, 128, GATE>(a, L, I, N, stream)
                          : launch_wave<64, 128, GATE>(a, L, I, N, stream);
    return D_k == 128 ? launch_wave<128, 64, GATE>(a, L, I, N, stream)
                      : launch_wave<64, 64, GATE>(a, L, I, N, stream);
}

// Waves of the T = 1 wave form with 64-column tiles that the current device holds at once.
static int wave_resident_64(int D_k, int gate) {
    if (D_k == 128)
        return gate == kGateGiven ? resident_waves<128, 64, kGateGiven>()
               : gate == kGateF32 ? resident_waves<128, 64, kGateF32>()
                                  : resident_waves<128, 64, kGateF16>();
    return gate == kGateGiven ? resident_waves<64, 64, kGateGiven>()
           : gate == kGateF32 ? resident_waves<64, 64, kGateF32>()
                              : resident_waves<64, 64, kGateF16>();
}

// Shape and alignment checks shared by both entry points, then the launch of the form that
// T and the head sizes pick.
static rgdr_status decode_entry(DecodeArgs &a, int gate, int32_t B, int32_t H_q, int32_t H_v,
                                int32_t T, int32_t D_k, int32_t D_v, int32_t N_slots,
                                const int32_t *lens, const int32_t *idx, const int32_t *nacc,
                                hipStream_t stream) {
    if (B < 0 || H_q <= 0 || H_v <= 0 || T <= 0 || D_k <= 0 || D_v <= 0 || N_slots <= 0)
        return RGDR_ERR_SHAPE;
    if (T > kMaxT || H_v % H_q != 0) return RGDR_ERR_SHAPE;
    if ((D_k != 64 && D_k != 128) || D_v % 64 != 0 || D_v > 4096) return RGDR_ERR_UNSUPPORTED;
    if (!aligned(a.v, 16) || !aligned(a.pool, 16) || !aligned(a.out, 16) ||
        !aligned(a.pool_out, 16) || !aligned(a.q, 16) || !aligned(a.k, 16) ||
        !aligned(a.gk, 16) || !aligned(lens, 4) || !aligned(idx, 4) || !aligned(nacc, 4) ||
        !aligned(a.snap, 16))
        return RGDR_ERR_ALIGN;
    const bool chunk = RGDR_CHUNK_FORM && T >= RGDR_CHUNK_MIN_T &&
                       (D_k == 128 || (RGDR_CHUNK_DK64 && T >= RGDR_CHUNK_DK64_MIN_T)) &&
                       (D_v % 128 == 0 ||
                        (RGDR_CHUNK_HALF_TILE && (D_v > 64 || T >= RGDR_CHUNK_DV64_MIN_T)));
    // Per-token states: the chunk form where it serves the call, else the per-token form
    // (also for T = 1: the single-token form keeps no snapshot path).
    const Form form = T == 1 && !a.snap ? kFormWave : chunk ? kFormChunk : kFormWaveMulti;
    // Tile widths. For the multi-token form, the widest tile whose fp32 copy fits a lane
    // (D_k x TV <= 64 x 128 values per wave). For T = 1, 64-column tiles while the whole call
    // then fits in one launch of the resident grid: twice the waves, each with half the
    // bytes and half the arithmetic, shorten a launch whose waves are not limited by the
    // memory system's rate (at H_v = 32, D = 128: 5.4 against 7.6 us at B = 1, 9.1 against
    // 10.6 at B = 16, 12.9 against 15.2 at B = 32). Past that, whole 256-byte rows (128
    // columns) when D_v allows: at B = 48 the narrow tiles need two launches (21.8 against
    // 19.2 us), and at B = 64 they stream worse (25.7 against 23.1 us).
    int tile_v = form == kFormChunk ? 128 : 64;
    if (form == kFormWaveMulti && D_k == 64 && D_v % 128 == 0) tile_v = 128;
    if (form == kFormWave && RGDR_WAVE_TILE_V == 128 && D_v % 128 == 0) {
        const int resident = wave_resident_64(D_k, gate);
        if (resident <= 0) return RGDR_ERR_HIP;
        if ((long long)B * H_v * (D_v / 64) > resident) tile_v = 128;
    }
    const int ntiles = (D_v + tile_v - 1) / tile_v;  // the chunk form's last tile may be half
    const long long items = (long long)B * H_v * ntiles;
    if (items > 0x7FFFFFFFLL) return RGDR_ERR_SHAPE;
    a.Hq = H_q;
    a.Hv = H_v;
    a.T = T;
    a.Dv = D_v;
    a.N_slots = N_slots;
    a.ntiles = ntiles;
    a.group = H_v / H_q;
    a.n_items = (int)items;
    hipError_t err;
    if (gate == kGateGiven)
        err = dispatch<kGateGiven>(a, D_k, tile_v, form, lens, idx, nacc, stream);
    else if (gate == kGateF32)
        err = dispatch<kGateF32>(a, D_k, tile_v, form, lens, idx, nacc, stream);
    else
        err = dispatch<kGateF16>(a, D_k, tile_v, form, lens, idx, nacc, stream);
    return err == hipSuccess ? RGDR_OK : RGDR_ERR_HIP;
}

}  // namespace rgdr

extern "C" rgdr_status rgdr_decode(const void *query, const void *key, const void *value,
                                   const void *beta, const void *state_pool,
                                   const int32_t *actual_seq_lengths,
                                   const int32_t *ssm_state_indices, const float *g,
                                   const float *gk, const int32_t *num_accepted_tokens,
                                   float scale, int32_t B, int32_t H_q, int32_t H_v, int32_t T,
                                   int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
                                   void *state_out, hipStream_t stream) {
    using namespace rgdr;
    if (B == 0) return RGDR_OK;  // empty batch: nothing to do, no pointer is read
    if (!query || !key || !value || !beta || !state_pool || !actual_seq_lengths ||
        !ssm_state_indices || !g || !gk || !num_accepted_tokens || !out || !state_out)
        return RGDR_ERR_NULL;
    if (!aligned(beta, 2) || !aligned(g, 4)) return RGDR_ERR_ALIGN;
    DecodeArgs a = {};
    a.q = static_cast<const uint16_t *>(query);
    a.k = static_cast<const uint16_t *>(key);
    a.v = static_cast<const uint16_t *>(value);
    a.beta = static_cast<const uint16_t *>(beta);
    a.pool = static_cast<const uint16_t *>(state_pool);
    a.g = g;
    a.gk = gk;
    a.out = static_cast<uint16_t *>(out);
    a.pool_out = static_cast<uint16_t *>(state_out);
    a.scale = scale;
    return decode_entry(a, kGateGiven, B, H_q, H_v, T, D_k, D_v, N_slots, actual_seq_lengths,
                        ssm_state_indices, num_accepted_tokens, stream);
}

extern "C" rgdr_status rgdr_decode_snapshots(
    const void *query, const void *key, const void *value, const void *beta,
    const void *state_pool, const int32_t *actual_seq_lengths, const int32_t *ssm_state_indices,
    const float *g, const float *gk, const int32_t *num_accepted_tokens, float scale,
    int32_t B, int32_t H_q, int32_t H_v, int32_t T, int32_t D_k, int32_t D_v, int32_t N_slots,
    void *out, void *state_out, void *state_snapshots, hipStream_t stream) {
    using namespace rgdr;
    if (B == 0) return RGDR_OK;
    if (!query || !key || !value || !beta || !state_pool || !actual_seq_lengths ||
        !ssm_state_indices || !g || !gk || !num_accepted_tokens || !out || !state_out ||
        !state_snapshots)
        return RGDR_ERR_NULL;
    if (!aligned(beta, 2) || !aligned(g, 4)) return RGDR_ERR_ALIGN;
    DecodeArgs a = {};
    a.q = static_cast<const uint16_t *>(query);
    a.k = static_cast<const uint16_t *>(key);
    a.v = static_cast<const uint16_t *>(value);
    a.beta = static_cast<const uint16_t *>(beta);
    a.pool = static_cast<const uint16_t *>(state_pool);
    a.g = g;
    a.gk = gk;
    a.out = static_cast<uint16_t *>(out);
    a.pool_out = static_cast<uint16_t *>(state_out);
    a.snap = static_cast<uint16_t *>(state_snapshots);
    a.scale = scale;
    return decode_entry(a, kGateGiven, B, H_q, H_v, T, D_k, D_v, N_slots, actual_seq_lengths,
                        ssm_state_indices, num_accepted_tokens, stream);
}

namespace rgdr {
// Argument checks and marshalling shared by the two fused-gate decode entries.
static rgdr_status decode_gated(const void *query, const void *key, const void *value,
                                const void *gate_a, const void *gate_b, const float *dt_bias,
                                const float *decay_scale, rgdr_dtype gate_dtype,
                                const void *state_pool, const int32_t *actual_seq_lengths,
                                const int32_t *ssm_state_indices, const float *gk,
                                const int32_t *num_accepted_tokens, float scale, int32_t B,
                                int32_t H_q, int32_t H_v, int32_t T, int32_t D_k, int32_t D_v,
                                int32_t N_slots, void *out, void *state_out, void *snap,
                                bool snap_required, uint32_t flags, hipStream_t stream) {
    if (flags & ~(uint32_t)RGDR_NORMALIZE_QK) return RGDR_ERR_UNSUPPORTED;
    if (B == 0) return RGDR_OK;
    if (!query || !key || !value || !gate_a || !gate_b || !dt_bias || !decay_scale ||
        !state_pool || !actual_seq_lengths || !ssm_state_indices || !gk ||
        !num_accepted_tokens || !out || !state_out || (snap_required && !snap))
        return RGDR_ERR_NULL;
    if (gate_dtype != RGDR_F32 && gate_dtype != RGDR_F16) return RGDR_ERR_DTYPE;
    const uintptr_t esz = gate_dtype == RGDR_F16 ? 2 : 4;
    if (!aligned(gate_a, esz) || !aligned(gate_b, esz) || !aligned(dt_bias, 4) ||
        !aligned(decay_scale, 4))
        return RGDR_ERR_ALIGN;
    DecodeArgs a = {};
    a.q = static_cast<const uint16_t *>(query);
    a.k = static_cast<const uint16_t *>(key);
    a.v = static_cast<const uint16_t *>(value);
    a.pool = static_cast<const uint16_t *>(state_pool);
    a.gk = gk;
    a.ga = gate_a;
    a.gb = gate_b;
    a.dt_bias = dt_bias;
    a.dscale = decay_scale;
    a.norm_qk = (flags & RGDR_NORMALIZE_QK) ? 1 : 0;
    a.out = static_cast<uint16_t *>(out);
    a.pool_out = static_cast<uint16_t *>(state_out);
    a.snap = static_cast<uint16_t *>(snap);
    a.scale = scale;
    return decode_entry(a, gate_dtype == RGDR_F16 ? kGateF16 : kGateF32, B, H_q, H_v, T, D_k,
                        D_v, N_slots, actual_seq_lengths, ssm_state_indices,
                        num_accepted_tokens, stream);
}
}  // namespace rgdr

extern "C" rgdr_status rgdr_decode_gated(const void *query, const void *key, const void *value,
                                         const void *gate_a, const void *gate_b,
                                         const float *dt_bias, const float *decay_scale,
                                         rgdr_dtype gate_dtype, const void *state_pool,
                                         const int32_t *actual_seq_lengths,
                                         const int32_t *ssm_state_indices, const float *gk,
                                         const int32_t *num_accepted_tokens, float scale,
                                         int32_t B, int32_t H_q, int32_t H_v, int32_t T,
                                         int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
                                         void *state_out, uint32_t flags, hipStream_t stream) {
    return rgdr::decode_gated(query, key, value, gate_a, gate_b, dt_bias, decay_scale,
                              gate_dtype, state_pool, actual_seq_lengths, ssm_state_indices, gk,
                              num_accepted_tokens, scale, B, H_q, H_v, T, D_k, D_v, N_slots, out,
                              state_out, nullptr, false, flags, stream);
}

extern "C" rgdr_status rgdr_decode_gated_snapshots(
    const void *query, const void *key, const void *value, const void *gate_a,
    const void *gate_b, const float *dt_bias, const float *decay_scale, rgdr_dtype gate_dtype,
    const void *state_pool, const int32_t *actual_seq_lengths, const int32_t *ssm_state_indices,
    const float *gk, const int32_t *num_accepted_tokens, float scale, int32_t B, int32_t H_q,
    int32_t H_v, int32_t T, int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
    void *state_out, void *state_snapshots, uint32_t flags, hipStream_t stream) {
    return rgdr::decode_gated(query, key, value, gate_a, gate_b, dt_bias, decay_scale,
                              gate_dtype, state_pool, actual_seq_lengths, ssm_state_indices, gk,
                              num_accepted_tokens, scale, B, H_q, H_v, T, D_k, D_v, N_slots, out,
                              state_out, state_snapshots, true, flags, stream);
}
