// rgdr_prefill.hip -- the gated-delta recurrence over long sequences (T > 8) on gfx950.
//
// Method: MindSpore Lite API page "lite_boost.ops.recurrent_gated_delta_rule". Its
// algorithm section gives the four steps applied token by token; its notes limit that
// decode operator to T <= 8 and send the parallel prefill to a chunk-level operator. This
// is that operator for this library: the same inputs, outputs and semantics as rgdr_decode
// (slot pool, lengths, accepted counts, head sharing, padding), for any T up to 65536.
//
// Design. One workgroup of four waves owns one (entry, value head, column tile) for the
// whole sequence: 128 columns, or 256 at D_k = 64 when a call has more items than the device
// holds at once, or 64 at D_k = 128 when it leaves most compute units idle. Its state tile is read from HBM once, kept in fp32 in the matrix cores'
// accumulator layout while the item's tokens are walked in chunks of up to 32, and written
// back once (at the accepted prefix's end). Each chunk applies the exact closed form of the
// four steps over its tokens (the unrolled recurrence the decode kernel's chunk form also
// uses), with the state S0 at the chunk's start:
//   d_t = exp(g_t) exp(gk_t) (per row), c_t = d_1 ... d_t (c_0 = 1), S' = diag(d_0) S0,
//   Y_K = [c k]^T S',  Y_Q = [c scale q]^T S',
//   M[t][s] = sum_i (c_t / c_s)_i k_t,i k_s,i (s < t),  N[t][s] = the same with scale q_t (s <= t),
//   (I + diag(beta) M) U = diag(beta) (V - Y_K),   O = Y_Q + N U,
//   S_end = diag(c_last) S' + sum_s diag(c_last / c_s) k_s u_s^T = diag(c_last) (S' + K_D^T U),
// with K_D the rows k_s / c_s. The registers hold S' + K_D^T U; c_last scales it into the next
// chunk's S' (with that chunk's d_0) or into the committed state.
// The two products with S' and the rank-32 update are matrix-core products on the state's
// own accumulator registers; M and N are matrix-core products of the factors c_t k_t (or
// c_t scale q_t) and k_s / c_s; the 32 x 32 triangular system is solved blockwise: the two
// 16 x 16 diagonal blocks are inverted by forward substitution in fp32 (one wave each), and
//   U_0 = A_00 R_0,   U_1 = A_11 (R_1 - M_10 U_0),   A_bb = (I + diag(beta) M_bb)^-1 diag(beta)
// are matrix-core products. Every fp32 operand of a matrix-core product is split into a bf16
// high part and a bf16 remainder and three products are summed (high x high, low x high,
// high x low), so each keeps about 16 bits of both operands; accumulation is fp32.
//
// The closed form holds with c measured from any per-row reference: with c'_t = c_t / r and
// S'' = diag(r) S', Y_K = [c' k]^T S'', M and N take the ratios c'_t / c'_s = c_t / c_s, and
// S_end = diag(c'_last) (S'' + K'^T U) with K' the rows k_s / c'_s. Each row takes the
// middle of its chunk, r = 2^(L_last / 2) with L_t = log2 c_t (sums of the decays' log2,
// formed in log space so that no product under- or overflows), and the factored form needs
// every c'_t within [2^-96, 2^96]: a chunk whose decay products span up to 2^192. Each
// factor, and S'' (at most 2^96 times the state), then stays far from fp32's limits. Every
// pair the form keeps (s <= t) has c'_t / c'_s = c_t / c_s <= 1 in the operator's domain,
// so its products stay within the operands' size. The pairs above the diagonal may
// overflow: the forward substitution never reads them, and the N blocks replace them by
// zeros with a select, so an inf or NaN there never reaches a kept entry. A chunk in which some row leaves that range is shortened (a
// row's first token lies within it, so at least one token remains); strong decays
// therefore give shorter chunks, not a different arithmetic.
//
// A chunk that holds the accepted prefix's end stops there, so the committed state is a
// chunk's end state; the later tokens still produce their outputs. The next chunk's operands
// are loaded while the current one is computed. HBM sees the state once in and once out,
// and every operand once.
#include <atomic>
#include <climits>
#include <type_traits>

#include "rgdr_device.h"

namespace rgdr {

constexpr int kPrefillMaxT = 65536;  // tokens per call: keeps every per-item offset in 32 bits
constexpr int kChunk = 32;           // tokens per chunk
// Range (log2) of the decay products c'_t around the chunk's middle inside which a chunk takes
// the factored form.
constexpr float kChunkLog2 = 96.f;
constexpr float kLog2e = 1.4426950408889634f;  // exp(x) = 2^(x log2 e)

// The segmented form's workspace (a caller's, or the fixed array): each segment's transfer
// [Psi | Phi] fp32 [B, H_v, nseg, D_k, D_v + D_k], and each segment's incoming state fp32
// [B, H_v, nseg, D_k, D_v]; seg_len tokens per segment (a multiple of the chunk).
struct SegArgs {
    float *ws_e, *ws_s;
    int nseg, seg_len;
};

// Waves per SIMD the kernel is compiled for (the register budget).
#ifndef RGDR_PREFILL_MIN_WAVES
#define RGDR_PREFILL_MIN_WAVES 2
#endif

// Thread mapping and LDS carve of one item (256 threads).
//   Preparation: thread (r, tg) = (tid / NTG, tid % NTG) owns rows 4 r .. 4 r + 3 of tokens
//   TPT tg .. TPT tg + TPT - 1; the NTG token groups of a row group are consecutive lanes.
//   XK, XQ, KD: [hi, lo][32 tokens][XS] bf16: c_t k_t, c_t scale q_t, k_t / c_t by row.
//   KH: [hi, lo][D_k rows][KS] bf16: (c_last / c_s) k_s, one row per state row.
//   TD: [2][16][BS] fp32: beta_t M[t][s] of the two diagonal 16 x 16 blocks, by column s.
//   BK: [6 blocks][hi, lo][16][AS] bf16: A_00, A_11, -M_10, N_00, N_10, N_11.
//   c_last and d_0 per row, beta per token, and the chunk cut.
template <int DK>
struct ChunkShape {
    static constexpr int NRB = DK / 16, NPB = DK / 32;
    static constexpr int TPT = DK / 32;       // tokens per preparing thread
    static constexpr int NTG = kChunk / TPT;  // token groups: lanes per row group
    static_assert((DK / 4) * NTG == 256, "four rows by TPT tokens per thread");
    static_assert(NTG == 8 || NTG == 16, "token groups inside one 16-lane DPP row");
    static constexpr int XS = DK + 4, KS = kChunk + 4, AS = 16 + 4, BS = 16 + 4;
    // The small, often-addressed areas come first, so that every access below 64 KiB takes
    // its constant part in the LDS instruction's 16-bit offset; KD, read only by the M and N
    // products, comes last.
    static constexpr int XBYTES = 2 * kChunk * XS * 2;
    static constexpr int OFF_CUT = 0;
    static constexpr int OFF_BT = 16;
    static constexpr int OFF_D0 = OFF_BT + kChunk * 4;
    static constexpr int OFF_CL = OFF_D0 + DK * 4;
    static constexpr int OFF_TD = OFF_CL + DK * 4;
    static constexpr int OFF_BK = OFF_TD + 2 * 16 * BS * 4;
    static constexpr int OFF_KH = OFF_BK + 6 * 2 * 16 * AS * 2;
    static constexpr int OFF_XK = OFF_KH + 2 * DK * KS * 2;
    static constexpr int OFF_XQ = OFF_XK + XBYTES;
    static constexpr int OFF_KD = OFF_XQ + XBYTES;
    static constexpr int BYTES = OFF_KD + XBYTES;
    static_assert(BYTES % 16 == 0 && BYTES <= 81920, "LDS carve: two items per compute unit");
    // The q/k norm partials [4 waves][2][32] (preparation only) share the TD area.
    static_assert(4 * 2 * kChunk * 4 <= 2 * 16 * BS * 4, "norm partials fit TD");
};

// One chunk's operands in flight: this thread's rows of k, q and gk for its tokens, and the
// gate values of token lane % 32.
template <int DK>
struct ChunkOps {
    static constexpr int TPT = ChunkShape<DK>::TPT;
    u32x2 k[TPT], q[TPT];
    f32x4 gk[TPT];
    uint32_t ga, gb;  // g (fp32) and beta (bf16), or the raw gate projections a and b
};

// Issue the loads of tokens t0 .. t0 + len - 1 (ranges stop at len: later tokens read zeros).
template <int DK, int GATE>
__device__ __forceinline__ void load_chunk(const DecodeArgs &a, const Item &m, ChunkOps<DK> &o,
                                           int r, int tg, int lane, int t0, int len) {
    constexpr int TPT = ChunkShape<DK>::TPT;
    const size_t bhT = ((size_t)m.b * a.Hv + m.h) * a.T + t0;
    const size_t qk0 = (((size_t)m.b * a.Hq + m.hq) * a.T + t0) * DK;
    const uint32_t n = (uint32_t)len;
    const auto rk = make_rsrc(a.k + qk0, n * DK * 2);
    const auto rq = make_rsrc(a.q + qk0, n * DK * 2);
    const auto rgk = make_rsrc(a.gk + bhT * DK, n * DK * 4);
    const uint32_t e = (uint32_t)(TPT * tg * DK + 4 * r);
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
        o.k[j] = __builtin_amdgcn_raw_buffer_load_b64(rk, e * 2, j * DK * 2, 0);
        o.q[j] = __builtin_amdgcn_raw_buffer_load_b64(rq, e * 2, j * DK * 2, 0);
        o.gk[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rgk, e * 4, j * DK * 4, 0));
    }
    const int t = lane & 31;
    if constexpr (GATE == kGateGiven) {
        o.ga = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.g + bhT, n * 4), t * 4, 0, 0);
        o.gb = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(a.beta + bhT, n * 2), t * 2, 0, 0);
    } else {
        o.ga = gate_raw(a, a.ga, GATE, m.b, t0 + t, m.h, t < len);
        o.gb = gate_raw(a, a.gb, GATE, m.b, t0 + t, m.h, t < len);
    }
}

// f32x4 -> bf16 high parts and bf16 remainders (x - hi is exact in fp32), packed in order.
__device__ __forceinline__ void split4(const f32x4 &x, uint2 &hi, uint2 &lo) {
    hi.x = pack_bf16x2(x.x, x.y);
    hi.y = pack_bf16x2(x.z, x.w);
    lo.x = pack_bf16x2(x.x - bf16_lo(hi.x), x.y - bf16_hi(hi.x));
    lo.y = pack_bf16x2(x.z - bf16_lo(hi.y), x.w - bf16_hi(hi.y));
}
// f32x4 pair -> the same, 8 values in k order (x0 first).
__device__ __forceinline__ void split8(const f32x4 &x0, const f32x4 &x1, bf16x8 &hi, bf16x8 &lo) {
    uint2 h0, l0, h1, l1;
    split4(x0, h0, l0);
    split4(x1, h1, l1);
    hi = __builtin_bit_cast(bf16x8, u32x4{h0.x, h0.y, h1.x, h1.y});
    lo = __builtin_bit_cast(bf16x8, u32x4{l0.x, l0.y, l1.x, l1.y});
}
__device__ __forceinline__ s16x4 as_s16x4(uint2 v) { return __builtin_bit_cast(s16x4, v); }

// NC consecutive bf16 columns of one row (1, 2 or 4) in one buffer access, as (NC + 1) / 2
// 32-bit words (one column: the low half).
template <int NC, int POL>
__device__ __forceinline__ void load_cols(uint32_t (&w)[(NC + 1) / 2], __amdgpu_buffer_rsrc_t rs,
                                          uint32_t voff, uint32_t soff) {
    if constexpr (NC == 1) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, POL);
    } else if constexpr (NC == 2) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, POL);
    } else {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, POL);
        w[0] = v.x;
        w[1] = v.y;
    }
}
template <int NC, int POL>
__device__ __forceinline__ void store_cols(const uint32_t (&w)[(NC + 1) / 2],
                                           __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                           uint32_t soff) {
    if constexpr (NC == 1)
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w[0], rs, voff, soff, POL);
    else if constexpr (NC == 2)
        __builtin_amdgcn_raw_buffer_store_b32(w[0], rs, voff, soff, POL);
    else
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, rs, voff, soff, POL);
}
// NC consecutive fp32 columns of one row in one buffer access (the segmented form's
// workspace).
template <int NC>
__device__ __forceinline__ void load_cols_f32(float (&v)[NC], __amdgpu_buffer_rsrc_t rs,
                                              uint32_t voff, uint32_t soff) {
    if constexpr (NC == 1) {
        v[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0));
    } else if constexpr (NC == 2) {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
        v[0] = __uint_as_float(x.x);
        v[1] = __uint_as_float(x.y);
    } else {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = __uint_as_float(x[c]);
    }
}
template <int NC>
__device__ __forceinline__ void store_cols_f32(const float (&v)[NC], __amdgpu_buffer_rsrc_t rs,
                                               uint32_t voff, uint32_t soff) {
    if constexpr (NC == 1) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), rs, voff, soff, 0);
    } else if constexpr (NC == 2) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v[0]), __float_as_uint(v[1])},
                                              rs, voff, soff, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                  __float_as_uint(v[3])},
            rs, voff, soff, 0);
    }
}
__device__ __forceinline__ bf16x8 cat8(uint2 a, uint2 b) {
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// 16 x 16 block G[t][s] = sum_i A[16 tb + t][i] B[16 sb + s][i] over the D_k rows of two
// [hi, lo][32][XS] operand planes, three products of the split parts. Lane (kg, n16) ends with
// G[4 kg + i][n16]. The k slots of lane group kg are columns 4 kg .. + 3 and 16 + 4 kg .. + 3
// of each 32-column group (the same order on both sides).
template <int DK, int XS>
__device__ __forceinline__ f32x4 gram_block(const uint16_t *a_hi, const uint16_t *b_hi, int tb,
                                            int sb, int n16, int kg) {
    const uint16_t *a_lo = a_hi + kChunk * XS, *b_lo = b_hi + kChunk * XS;
    f32x4 g = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pb = 0; pb < DK / 32; ++pb) {
        const int ra = (16 * tb + n16) * XS + 32 * pb + 4 * kg;
        const int rb = (16 * sb + n16) * XS + 32 * pb + 4 * kg;
        const bf16x8 ah = lds_pair8(a_hi + ra, a_hi + ra + 16), al = lds_pair8(a_lo + ra, a_lo + ra + 16);
        const bf16x8 bh = lds_pair8(b_hi + rb, b_hi + rb + 16), bl = lds_pair8(b_lo + rb, b_lo + rb + 16);
        g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, g, 0, 0, 0);
        g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, g, 0, 0, 0);
        g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, g, 0, 0, 0);
    }
    return g;
}

// A 16 x 16 accumulator block (lane (kg, n16): rows 4 kg + i, column n16) into an operand
// block [hi, lo][16][AS], entries with column > row zeroed when LOWER.
template <int AS, bool LOWER>
__device__ __forceinline__ void put_block(uint16_t *blk, const f32x4 &g, float sign, int n16, int kg) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * kg + i;
        const float v = (!LOWER || n16 <= row) ? sign * g[i] : 0.f;
        uint16_t h, l;
        split_bf16(v, h, l);
        blk[row * AS + n16] = h;
        blk[16 * AS + row * AS + n16] = l;
    }
}

// One 16x16x16 product chain of split operands: acc + A x B (high x high, low x high, high x low).
__device__ __forceinline__ f32x4 mma16(s16x4 ah, s16x4 al, s16x4 bh, s16x4 bl, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
}

// Lane layout of the state. Wave w owns the WC = 16 NC tile columns WC w .. WC w + WC - 1
// over all D_k rows (NC = 2: 128-column tiles; NC = 4: 256-column tiles, D_k = 64 only, where
// the state still takes 64 values per lane; NC = 1: 64-column tiles, D_k = 128 only, for
// calls with few items). Lane l = (kg, n16) = (l / 16, l % 16) holds rows
// 16 rb + 4 kg + i (rb < D_k / 16, i < 4) of columns WC w + NC n16 + c (c < NC) as
// S[rb][c][i]: the accumulator layout of the 16 x 16 block of rows 16 rb .. + 15 and columns
// WC w + NC n + c (column set c). Rows 4 kg .. 4 kg + 3 of two
// row blocks are also the 8 k slots of lane group kg in a 16x16x32 product, so the state turns
// into the B operand of Y = X S in the lane that holds it. The chunk's per-token results (Y_K,
// Y_Q, U, O) use the same layout with tokens for rows: 16 tb + 4 kg + i is the token, and the
// rows 4 kg .. + 3 of a 16-token block are the k slots of a 16x16x16 product over tokens.
//
// SEG selects the form. 0: the single pass above. The segmented form cuts each entry's tokens
// into segments (at the accepted count too) and runs the kernel twice over all segments at
// once, with a sequential scan between (prefill_scan_kernel). Every state column follows the
// recurrence on its own, with its own column of v, so a segment maps its incoming state S to
// Phi S + Psi: Psi is the end state from zero, and the columns of Phi are the end states of
// the identity's columns with v = 0. SEG = 1 evaluates both at once, as D_v + D_k columns,
// and stores them in fp32; SEG = 2 starts each segment from its true incoming state (fp32,
// from the scan) and writes the outputs. Neither reads nor commits the pool; the scan does.
template <int DK, int GATE, bool NORM, int NC, int SEG = 0>
__global__ __launch_bounds__(256, RGDR_PREFILL_MIN_WAVES) void prefill_kernel(
    const DecodeArgs a, const int32_t *__restrict__ lens, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nacc, const SegArgs sg) {
    static_assert(DK == 64 || DK == 128, "D_k = 64 or 128");
    static_assert(!NORM || GATE != kGateGiven, "q/k normalisation belongs to the fused front end");
    static_assert(NC == 2 || (NC == 4 && DK == 64) || (NC == 1 && DK == 128),
                  "256-column tiles at D_k = 64 only, 64-column tiles at D_k = 128 only");
    using P = ChunkShape<DK>;
    constexpr int WC = 16 * NC, TV = 4 * WC, NW = (NC + 1) / 2;  // NW: words per lane row
    constexpr int NRB = P::NRB, NPB = P::NPB, TPT = P::TPT, NTG = P::NTG;
    constexpr int XS = P::XS, KS = P::KS, AS = P::AS, BS = P::BS;
    __shared__ f32x4 lds4[P::BYTES / 16];
    char *lb = reinterpret_cast<char *>(lds4);
    uint16_t *xk_hi = reinterpret_cast<uint16_t *>(lb + P::OFF_XK), *xk_lo = xk_hi + kChunk * XS;
    uint16_t *xq_hi = reinterpret_cast<uint16_t *>(lb + P::OFF_XQ), *xq_lo = xq_hi + kChunk * XS;
    uint16_t *kd_hi = reinterpret_cast<uint16_t *>(lb + P::OFF_KD), *kd_lo = kd_hi + kChunk * XS;
    uint16_t *kh_hi = reinterpret_cast<uint16_t *>(lb + P::OFF_KH), *kh_lo = kh_hi + DK * KS;
    float *td = reinterpret_cast<float *>(lb + P::OFF_TD);
    float *npart = td;
    uint16_t *bk = reinterpret_cast<uint16_t *>(lb + P::OFF_BK);
    float *crow = reinterpret_cast<float *>(lb + P::OFF_CL);
    float *d0row = reinterpret_cast<float *>(lb + P::OFF_D0);
    float *bt = reinterpret_cast<float *>(lb + P::OFF_BT);
    int *cut = reinterpret_cast<int *>(lb + P::OFF_CUT);
    auto blk = [&](int b) { return bk + b * 2 * 16 * AS; };  // block b: hi, then lo at + 16 AS

    const Index x{lens, idx, nacc};
    const int tid = threadIdx.x, lane = tid & 63, n16 = lane & 15, kg = lane >> 4;
    // w is the same in every lane of a wave; readfirstlane tells the compiler so, which keeps
    // the buffer descriptors built from it in scalar registers.
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = tid / NTG, tg = tid % NTG;  // preparation: rows 4 r .. + 3, tokens TPT tg ..
    // Items (entry, value head, tile), or (entry, value head, segment, tile) when segmented.
    int it = xcd_item(blockIdx.x, gridDim.x), seg = 0;
    if constexpr (SEG != 0) {
        const int tl = it % a.ntiles, rest = it / a.ntiles;
        seg = rest % sg.nseg;
        it = (rest / sg.nseg) * a.ntiles + tl;
    }
    const Item m = resolve(a, x, it);
    const int L = m.L, n = m.n;
    // Tokens tbeg .. tend - 1 of the entry; the chunk holding ncut (the accepted prefix's
    // end) stops there. A segment is seg_len tokens of [0, n), or of [n, L) after the
    // ceil(n / seg_len) segments of the prefix.
    int tbeg = 0, tend = L, ncut = n;
    if constexpr (SEG != 0) {
        const int sl = sg.seg_len, na = (n + sl - 1) / sl;
        tbeg = seg < na ? seg * sl : n + (seg - na) * sl;
        tend = min(tbeg + sl, seg < na ? n : L);
        if (tbeg >= tend) {  // an empty segment: only the first segment's outputs remain
            if (SEG == 1 || seg != 0) return;
            tbeg = tend = 0;
        }
        ncut = tend;
    }
    // Columns: D_v state columns, then (SEG = 1) the D_k columns of Phi.
    const int ncols = SEG == 1 ? a.Dv + DK : a.Dv;
    const int colw = m.tile * TV + WC * w;  // this wave's first column
    const bool phi = SEG == 1 && colw >= a.Dv;  // a wave's columns are all of Psi or of Phi

    // A narrower last tile (D_v not a multiple of the tile) leaves the waves past D_v without
    // columns: their state, value and output accesses get empty ranges and they compute on
    // zeros.
    const bool cols = colw < ncols;
    const uint32_t trange = cols ? tile_range<DK, TV>(a, m) : 0u;
    const size_t tb0 = m.state ? tile_base<DK, TV>(a, m) : 0;
    const auto rs = make_rsrc(a.pool + tb0, trange);
    const auto rso = make_rsrc(a.pool_out + tb0, trange);
    const uint32_t lane_off = (uint32_t)((4 * kg * a.Dv + WC * w + NC * n16) * 2);
    const size_t bh = (size_t)m.b * a.Hv + m.h;
    const uint32_t ocol = (uint32_t)((m.tile * TV + WC * w + NC * n16) * 2);
    // Token (or state row) 4 kg + i of a 16-row block: the lane's part in the vector offset,
    // the rest in the scalar one (4- and 8-byte accesses only; see store16 for the wide ones).
    const uint32_t orow = ocol + (uint32_t)(4 * kg * a.Dv * 2);
    float dt = 0.f, ds = 0.f;
    if constexpr (GATE != kGateGiven) gate_head(a, m.h, dt, ds);

    // Chunks of at most kChunk tokens; the chunk holding the accepted prefix's end stops there.
    auto chunk_len = [&](int t0) {
        const int t1 = min(t0 + kChunk, tend);
        return ((t0 < ncut && ncut < t1) ? ncut : t1) - t0;
    };
    // This lane's values of tokens 16 tb + 4 kg + i, columns WC w + NC n16 + (0 .. NC - 1).
    uint32_t vr[2][4][NW];
    auto load_v = [&](int t0, int len) {
        const auto rv = make_rsrc(a.v + (bh * a.T + t0) * a.Dv,
                                  cols && !phi ? (uint32_t)(len * a.Dv * 2) : 0u);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                load_cols<NC, 0>(vr[tb][i], rv, orow, (uint32_t)((16 * tb + i) * a.Dv * 2));
    };

    // The first chunk's operands, then the state tile (bf16 -> fp32, exact).
    int t0 = tbeg, len = chunk_len(tbeg);
    ChunkOps<DK> o;
    load_chunk<DK, GATE>(a, m, o, r, tg, lane, t0, len);
    load_v(t0, len);
    f32x4 S[NRB][NC];
    // The segment's workspace rows (SEG != 0): [entry, head, segment][D_k rows][ncols] fp32.
    const size_t wrow0 = ((bh * sg.nseg + seg) * DK) * (size_t)ncols;
    const uint32_t wlane = (uint32_t)((4 * kg * ncols + colw + NC * n16) * 4);
    if constexpr (SEG == 1) {
        // Psi from zero; Phi from the identity (column D_v + j holds row j's unit vector)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    S[rb][c][i] = (colw + NC * n16 + c - a.Dv == 16 * rb + 4 * kg + i) ? 1.f : 0.f;
    } else if constexpr (SEG == 2) {
        const auto rsw = make_rsrc(sg.ws_s + wrow0, cols ? (uint32_t)(DK * ncols * 4) : 0u);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v[NC];
                load_cols_f32<NC>(v, rsw, wlane, (uint32_t)((16 * rb + i) * ncols * 4));
#pragma unroll
                for (int c = 0; c < NC; ++c) S[rb][c][i] = v[c];
            }
    } else {
        uint32_t raw[NRB][4][NW];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                load_cols<NC, RGDR_STATE_LOAD_POLICY>(raw[rb][i], rs, lane_off,
                                                      (uint32_t)((16 * rb + i) * a.Dv * 2));
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    S[rb][c][i] = (c & 1) ? bf16_hi(raw[rb][i][c >> 1]) : bf16_lo(raw[rb][i][c >> 1]);
        if (n == 0) {  // nothing accepted: commit the incoming bytes
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    store_cols<NC, RGDR_STATE_STORE_POLICY>(raw[rb][i], rso, lane_off,
                                                            (uint32_t)((16 * rb + i) * a.Dv * 2));
        }
    }
    if (tid == 0) *cut = kChunk;
    lds_barrier();

    // Preparation of one chunk of Lc tokens from the operands in o (tokens >= Lc were loaded
    // as zeros, or zeroed): per-token gate values, the decay products c, and the operand
    // planes XK, XQ, KD, KH with c_last and d_0 per row and beta per token. A row whose c leaves
    // the factored range lowers *cut to the first such token.
    auto prep = [&](int Lc, const f32x4 &cprev) {
        float gll, btl;  // lane t = lane % 32: g_t log2(e) and beta_t (neutral past Lc)
        {
            const int t = lane & 31;
            float g, bv;
            if constexpr (GATE == kGateGiven) {
                g = __uint_as_float(o.ga);
                bv = bf16_to_f32((uint16_t)o.gb);
            } else {
                g = ds * softplus_fast(gate_value<GATE == kGateF16>(o.ga) + dt);
                bv = sigmoid_fast(gate_value<GATE == kGateF16>(o.gb));
            }
            const bool in = t < Lc;
            gll = in ? g * kLog2e : 0.f;
            btl = in ? bv : 0.f;
        }
        if (w == 0 && lane < kChunk) bt[lane] = btl;
        float gl[TPT], ks[TPT], qs[TPT], kf[TPT][4], qf[TPT][4];
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            gl[j] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (TPT * tg + j), __float_as_int(gll)));
            kf[j][0] = bf16_lo(o.k[j].x);
            kf[j][1] = bf16_hi(o.k[j].x);
            kf[j][2] = bf16_lo(o.k[j].y);
            kf[j][3] = bf16_hi(o.k[j].y);
            qf[j][0] = bf16_lo(o.q[j].x);
            qf[j][1] = bf16_hi(o.q[j].x);
            qf[j][2] = bf16_lo(o.q[j].y);
            qf[j][3] = bf16_hi(o.q[j].y);
            ks[j] = 1.f;
            qs[j] = a.scale;
        }
        if constexpr (NORM) {  // L2-normalise each token's q and k over the D_k rows
            float sk[TPT], sq[TPT];
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                float a2 = 0.f, b2 = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a2 = fmaf(kf[j][e], kf[j][e], a2);
                    b2 = fmaf(qf[j][e], qf[j][e], b2);
                }
                sk[j] = colsum<NTG>(a2);  // over this wave's row groups (lanes NTG apart)
                sq[j] = colsum<NTG>(b2);
            }
            if (lane < NTG)
#pragma unroll
                for (int j = 0; j < TPT; ++j) {
                    npart[(2 * w) * kChunk + TPT * tg + j] = sk[j];
                    npart[(2 * w + 1) * kChunk + TPT * tg + j] = sq[j];
                }
            lds_barrier();
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                const int t = TPT * tg + j;
                float a2 = 0.f, b2 = 0.f;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    a2 += npart[(2 * v) * kChunk + t];
                    b2 += npart[(2 * v + 1) * kChunk + t];
                }
                ks[j] = inv_norm(a2);
                qs[j] = a.scale * inv_norm(b2);
            }
        }
        // log2 of the decays exp(g_t) exp(gk_t,i), and their running sums over this thread's
        // tokens (token 0 excluded): L_t = log2 c_t.
        float ld0[4], lc[TPT][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                const float l = fmaf(o.gk[j][e], kLog2e, gl[j]);
                if (j == 0) ld0[e] = l;
                acc += (j == 0 && tg == 0) ? 0.f : l;
                lc[j][e] = acc;
            }
        }
        // Across the row group's token groups: inclusive sums by DPP row shifts, then the
        // exclusive prefix (shift by one) and the chunk total (last token group).
        float inc[4], pre[4], llast[4], lref[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) inc[e] = lc[TPT - 1][e];
        auto shr = [](float v, auto k) {
            return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(0.f), __float_as_int(v),
                                                              0x110 + decltype(k)::value, 0xF, 0xF, false));
        };
#define RGDR_SCAN_STEP(K)                                                         \
    if constexpr (K < NTG) {                                                      \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                           \
            const float p = shr(inc[e], std::integral_constant<int, K>{});        \
            inc[e] = tg >= K ? inc[e] + p : inc[e];                               \
        }                                                                         \
    }
        RGDR_SCAN_STEP(1)
        RGDR_SCAN_STEP(2)
        RGDR_SCAN_STEP(4)
        RGDR_SCAN_STEP(8)
#undef RGDR_SCAN_STEP
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p = shr(inc[e], std::integral_constant<int, 1>{});
            pre[e] = tg >= 1 ? p : 0.f;
            llast[e] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (lane | (NTG - 1)), __float_as_int(inc[e])));
            lref[e] = 0.5f * llast[e];  // the row's reference: the middle of its chunk
        }
        // c'_t = 2^(L_t - L_ref); out-of-range (or NaN) exponents mark the chunk for a cut.
        float cp[TPT][4];
        bool out_of_range = false;
#pragma unroll
        for (int j = 0; j < TPT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lc[j][e] += pre[e];  // L_t of row 4 r + e
                const float x = lc[j][e] - lref[e];
                out_of_range |= !(x >= -kChunkLog2 && x <= kChunkLog2);
                cp[j][e] = __builtin_amdgcn_exp2f(x);
            }
        // Operand planes. Row-major by token for XK, XQ, KD; KH holds the same split values
        // as KD, by state row (its bf16 halves regrouped by byte permutes).
        uint2 dh[TPT], dl[TPT];
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const int t = TPT * tg + j;
            f32x4 vk, vq, vd;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float kk = NORM ? kf[j][e] * ks[j] : kf[j][e];
                vk[e] = cp[j][e] * kk;
                vq[e] = cp[j][e] * (qf[j][e] * qs[j]);
                vd[e] = kk * __builtin_amdgcn_rcpf(cp[j][e]);
            }
            uint2 h, l;
            const int off = t * XS + 4 * r;
            split4(vk, h, l);
            *reinterpret_cast<uint2 *>(xk_hi + off) = h;
            *reinterpret_cast<uint2 *>(xk_lo + off) = l;
            split4(vq, h, l);
            *reinterpret_cast<uint2 *>(xq_hi + off) = h;
            *reinterpret_cast<uint2 *>(xq_lo + off) = l;
            split4(vd, dh[j], dl[j]);
            *reinterpret_cast<uint2 *>(kd_hi + off) = dh[j];
            *reinterpret_cast<uint2 *>(kd_lo + off) = dl[j];
        }
        // Row 4 r + e of KH: the bf16 of row e from each token's packed pair (e even: low
        // halves, e odd: high halves).
        auto regroup = [](const uint2 (&v)[TPT], int e, int j0) {
            const uint32_t x1 = (e < 2) ? v[j0 + 1].x : v[j0 + 1].y, x0 = (e < 2) ? v[j0].x : v[j0].y;
            return __builtin_amdgcn_perm(x1, x0, (e & 1) ? 0x07060302u : 0x05040100u);
        };
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int off = (4 * r + e) * KS + TPT * tg;
            if constexpr (TPT == 4) {
                *reinterpret_cast<uint2 *>(kh_hi + off) = make_uint2(regroup(dh, e, 0), regroup(dh, e, 2));
                *reinterpret_cast<uint2 *>(kh_lo + off) = make_uint2(regroup(dl, e, 0), regroup(dl, e, 2));
            } else {
                *reinterpret_cast<uint32_t *>(kh_hi + off) = regroup(dh, e, 0);
                *reinterpret_cast<uint32_t *>(kh_lo + off) = regroup(dl, e, 0);
            }
        }
        // The state is kept as S'' + sum_s (k_s / c'_s) u_s^T, whose rows c'_last scales into
        // the true state: the next chunk's S'' takes c'_last (of this one) times its own d_0
        // and reference.
        if (tg == 0) {
            f32x4 cl, dr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cl[e] = __builtin_amdgcn_exp2f(llast[e] - lref[e]);
                dr[e] = cprev[e] * __builtin_amdgcn_exp2f(ld0[e] + lref[e]);
            }
            *reinterpret_cast<f32x4 *>(crow + 4 * r) = cl;
            *reinterpret_cast<f32x4 *>(d0row + 4 * r) = dr;
        }
        if (out_of_range) {  // rare: find where this row's chunk must end
            int first = kChunk;
#pragma unroll
            for (int j = TPT - 1; j >= 0; --j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // A row whose whole chunk spans more than 2^(2 * 96) ends before its first
                    // token beyond that span from the start (token 0 never is); otherwise
                    // before its first token out of range around the middle.
                    const bool wide = !(llast[e] >= -2.f * kChunkLog2 && llast[e] <= 2.f * kChunkLog2);
                    const float x = wide ? lc[j][e] : lc[j][e] - lref[e];
                    const float lim = wide ? 2.f * kChunkLog2 : kChunkLog2;
                    if (!(x >= -lim && x <= lim)) first = TPT * tg + j;
                }
            atomicMin(cut, first);
        }
    };

    int chunk = 0;
    while (t0 < tend) {  // uniform over the workgroup
        int Lc = len;
        // c_last of the previous chunk for this thread's rows (1 before the first chunk);
        // read once, since a second preparation pass rewrites crow
        const f32x4 cprev = (chunk == 0 || tg != 0) ? f32x4{1.f, 1.f, 1.f, 1.f}
                                                     : *reinterpret_cast<const f32x4 *>(crow + 4 * r);
        // Issue priority rises with the phase of the chunk (preparation 0, M and N blocks 1,
        // Y 2, the rest 3). Each SIMD holds a wave of each of the unit's two items, and the
        // wave further into its chunk goes first: its matrix-core chains stay fed while the
        // other item's preparation fills their gaps, instead of the two competing for issue
        // slots (one level for everything after the preparation: 4% faster; these four: 9%).
        __builtin_amdgcn_s_setprio(0);
        for (;;) {
            prep(Lc, cprev);
            lds_barrier();
            const int c = *cut;
            if (c >= Lc) break;
            // A decay product left the range at token c >= 1: the chunk ends before it.
            // Zero this thread's operands of the later tokens and prepare again. Nothing
            // written by the preparation is read before the barrier that ends it. The next
            // pass takes a new reference and, outside the operator's domain (growth mixed
            // with decay), may lower the cut again: every thread reads it before any can.
            lds_barrier();
            Lc = c;
#pragma unroll
            for (int j = 0; j < TPT; ++j)
                if (TPT * tg + j >= Lc) {
                    o.k[j] = u32x2{0u, 0u};
                    o.q[j] = u32x2{0u, 0u};
                    o.gk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
        const int t0n = t0 + Lc, lenn = t0n < tend ? chunk_len(t0n) : 0;

        __builtin_amdgcn_s_setprio(1);
        // M and N blocks, each wave its share (rotating by chunk so that the solves move
        // between the SIMDs): roles 0 and 1 form beta M of one diagonal block each and invert
        // it (in the same wave, so no barrier separates the steps); roles 2 and 3 form -M_10,
        // N_00, N_10 and N_11 as split operand blocks.
        const int role = (w + chunk) & 3;
        if (role < 2) {
            // beta M of diagonal block db = role, inverted by column-oriented forward
            // substitution (lane j < 16: column j; lanes 16..63 repeat and write nothing)
            const int db = role;
            const f32x4 mdd = gram_block<DK, XS>(xk_hi, kd_hi, db, db, n16, kg);
            float *tcol_w = td + db * 16 * BS;
#pragma unroll
            for (int i = 0; i < 4; ++i) tcol_w[n16 * BS + 4 * kg + i] = bt[16 * db + 4 * kg + i] * mdd[i];
            lds_phase();
            int jc = lane & 15;
            asm volatile("" : "+v"(jc));
            const float *tcol = td + db * 16 * BS;
            float xs[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) xs[rr] = rr == jc ? 1.f : 0.f;
#pragma unroll
            for (int c = 0; c < 15; ++c)
#pragma unroll
                for (int rr = c + 1; rr < 16; ++rr) xs[rr] = fmaf(-tcol[c * BS + rr], xs[c], xs[rr]);
            if (lane < 16) {
                const float bj = bt[16 * db + jc];
                uint16_t *ab = blk(db);
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    uint16_t h, l;
                    split_bf16(xs[rr] * bj, h, l);
                    ab[rr * AS + jc] = h;
                    ab[16 * AS + rr * AS + jc] = l;
                }
            }
        } else if (role == 2) {
            put_block<AS, false>(blk(2), gram_block<DK, XS>(xk_hi, kd_hi, 1, 0, n16, kg), -1.f, n16, kg);
            put_block<AS, true>(blk(3), gram_block<DK, XS>(xq_hi, kd_hi, 0, 0, n16, kg), 1.f, n16, kg);
        } else {
            put_block<AS, false>(blk(4), gram_block<DK, XS>(xq_hi, kd_hi, 1, 0, n16, kg), 1.f, n16, kg);
            put_block<AS, true>(blk(5), gram_block<DK, XS>(xq_hi, kd_hi, 1, 1, n16, kg), 1.f, n16, kg);
        }

        __builtin_amdgcn_s_setprio(2);
        // Y_K = [c k]^T S' and Y_Q = [c scale q]^T S' (32 tokens x this wave's 32 columns),
        // with S' = diag(d_0) S formed in place; three products of the split parts.
        f32x4 yk[2][NC], yq[2][NC];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int c = 0; c < NC; ++c) yk[tb][c] = yq[tb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 dv = *reinterpret_cast<const f32x4 *>(d0row + 16 * (2 * pb + h) + 4 * kg);
#pragma unroll
                for (int c = 0; c < NC; ++c) S[2 * pb + h][c] *= dv;
            }
            bf16x8 sh[NC], sl[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) split8(S[2 * pb][c], S[2 * pb + 1][c], sh[c], sl[c]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int ra = (16 * tb + n16) * XS + 32 * pb + 4 * kg;
                const bf16x8 kh = lds_pair8(xk_hi + ra, xk_hi + ra + 16), kl = lds_pair8(xk_lo + ra, xk_lo + ra + 16);
                const bf16x8 qh = lds_pair8(xq_hi + ra, xq_hi + ra + 16), ql = lds_pair8(xq_lo + ra, xq_lo + ra + 16);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    yk[tb][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, sh[c], yk[tb][c], 0, 0, 0);
                    yk[tb][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, sh[c], yk[tb][c], 0, 0, 0);
                    yk[tb][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, sl[c], yk[tb][c], 0, 0, 0);
                    yq[tb][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, sh[c], yq[tb][c], 0, 0, 0);
                    yq[tb][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, sh[c], yq[tb][c], 0, 0, 0);
                    yq[tb][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, sl[c], yq[tb][c], 0, 0, 0);
                }
            }
        }
        // The next chunk's operands travel while this one is finished.
        load_chunk<DK, GATE>(a, m, o, r, tg, lane, t0n, lenn);
        lds_barrier();  // every operand block is written
        if (tid == 0) *cut = kChunk;  // every thread read it before the barrier

        __builtin_amdgcn_s_setprio(3);
        // R = V - Y_K for the chunk's tokens (0 past Lc); then the next chunk's values.
        // (Written out per column pair: the loop form of these two statements schedules the
        // D_k = 128 kernel differently and measured 1.2% slower.)
        f32x4 R[2][NC];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                R[tb][0][i] = bf16_lo(vr[tb][i][0]) - yk[tb][0][i];
                if constexpr (NC >= 2) R[tb][1][i] = bf16_hi(vr[tb][i][0]) - yk[tb][1][i];
                if constexpr (NC == 4) {
                    R[tb][2][i] = bf16_lo(vr[tb][i][1]) - yk[tb][2][i];
                    R[tb][3][i] = bf16_hi(vr[tb][i][1]) - yk[tb][3][i];
                }
            }
        if (Lc < kChunk)  // uniform: a short chunk's later tokens (their values may be anything)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * tb + 4 * kg + i >= Lc) {
                        if constexpr (NC == 1)
                            R[tb][0][i] = 0.f;
                        else
                            R[tb][0][i] = R[tb][1][i] = 0.f;
                        if constexpr (NC == 4) R[tb][2][i] = R[tb][3][i] = 0.f;
                    }
        load_v(t0n, lenn);
        auto blk4 = [&](int b, int lo) {
            return as_s16x4(*reinterpret_cast<const uint2 *>(blk(b) + lo * 16 * AS + n16 * AS + 4 * kg));
        };
        // U_0 = A_00 R_0; U_1 = A_11 (R_1 - M_10 U_0); O = Y_Q + N U (each product its own
        // 16x16x16 chain; the sums with Y_Q on the VALU).
        uint2 u0h[NC], u0l[NC], u1h[NC], u1l[NC];
        f32x4 ov[2][NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            uint2 rh, rl;
            split4(R[0][c], rh, rl);
            const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
            const f32x4 u0 = mma16(blk4(0, 0), blk4(0, 1), as_s16x4(rh), as_s16x4(rl), z);
            split4(u0, u0h[c], u0l[c]);
            const f32x4 r1 = mma16(blk4(2, 0), blk4(2, 1), as_s16x4(u0h[c]), as_s16x4(u0l[c]), R[1][c]);
            split4(r1, rh, rl);
            const f32x4 u1 = mma16(blk4(1, 0), blk4(1, 1), as_s16x4(rh), as_s16x4(rl), z);
            split4(u1, u1h[c], u1l[c]);
            const f32x4 n0 = mma16(blk4(3, 0), blk4(3, 1), as_s16x4(u0h[c]), as_s16x4(u0l[c]), z);
            f32x4 n1 = mma16(blk4(4, 0), blk4(4, 1), as_s16x4(u0h[c]), as_s16x4(u0l[c]), z);
            n1 = mma16(blk4(5, 0), blk4(5, 1), as_s16x4(u1h[c]), as_s16x4(u1l[c]), n1);
            ov[0][c] = yq[0][c] + n0;
            ov[1][c] = yq[1][c] + n1;
        }
        if constexpr (SEG != 1) {
            // tokens past the chunk fall outside the output range and are not written
            const auto rout = make_rsrc(a.out + (bh * a.T + t0) * a.Dv, cols ? (uint32_t)(Lc * a.Dv * 2) : 0u);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t wo[NW];
#pragma unroll
                    for (int j = 0; j < NW; ++j) {
                        if constexpr (NC == 1)
                            wo[j] = pack_bf16x2(ov[tb][0][i], 0.f);
                        else
                            wo[j] = pack_bf16x2(ov[tb][2 * j][i], ov[tb][2 * j + 1][i]);
                    }
                    store_cols<NC, 0>(wo, rout, orow, (uint32_t)((16 * tb + i) * a.Dv * 2));
                }
        }
        // S = S' + KH^T U (the true state is diag(c_last) S), one 16x16x32 chain per block
        // over the chunk's tokens (k slots: tokens 4 kg .. + 3 of U_0, then of U_1).
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const int ra = (16 * rb + n16) * KS + 4 * kg;
            const bf16x8 ah = lds_pair8(kh_hi + ra, kh_hi + ra + 16), al = lds_pair8(kh_lo + ra, kh_lo + ra + 16);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                S[rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, cat8(u0h[c], u1h[c]), S[rb][c], 0, 0, 0);
                S[rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, cat8(u0h[c], u1h[c]), S[rb][c], 0, 0, 0);
                S[rb][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, cat8(u0l[c], u1l[c]), S[rb][c], 0, 0, 0);
            }
        }
        t0 = t0n;
        len = lenn;
        ++chunk;
        if (SEG == 1 && t0 == tend) {  // the segment's end state diag(c_last) S, in fp32
            const auto rsw = make_rsrc(sg.ws_e + wrow0, cols ? (uint32_t)(DK * ncols * 4) : 0u);
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const f32x4 cr = *reinterpret_cast<const f32x4 *>(crow + 16 * rb + 4 * kg);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v[NC];
#pragma unroll
                    for (int c = 0; c < NC; ++c) v[c] = S[rb][c][i] * cr[i];
                    store_cols_f32<NC>(v, rsw, wlane, (uint32_t)((16 * rb + i) * ncols * 4));
                }
            }
        }
        if (SEG == 0 && t0 == n) {  // the accepted prefix ends here: commit diag(c_last) S
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const f32x4 cr = *reinterpret_cast<const f32x4 *>(crow + 16 * rb + 4 * kg);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t ws[NW];
#pragma unroll
                    for (int j = 0; j < NW; ++j) {
                        if constexpr (NC == 1)
                            ws[j] = pack_bf16x2(S[rb][0][i] * cr[i], 0.f);
                        else
                            ws[j] = pack_bf16x2(S[rb][2 * j][i] * cr[i], S[rb][2 * j + 1][i] * cr[i]);
                    }
                    store_cols<NC, RGDR_STATE_STORE_POLICY>(ws, rso, lane_off,
                                                            (uint32_t)((16 * rb + i) * a.Dv * 2));
                }
            }
        }
        lds_barrier();  // the next chunk's preparation reuses every LDS area
    }

    // Padded (or skipped) tokens: +0.0 rows. Each lane stores 8 of the wave's WC columns of
    // one row, in groups of 64 / (WC / 8) rows; rows past T fall outside the range. (The
    // segmented form's first segment stores them.)
    if (cols && L < a.T && SEG != 1 && seg == 0) {
        constexpr int CG = WC / 8, RG = 64 / CG;  // 8-column groups per row, rows per store
        const int pad = a.T - L;
        const auto rz = make_rsrc(a.out + (bh * a.T + L) * a.Dv + m.tile * TV + WC * w,
                                  (uint32_t)(((pad - 1) * a.Dv + WC) * 2));
        const uint32_t ul = (uint32_t)lane;
        const uint32_t zoff = ((ul / CG) * (uint32_t)a.Dv + 8 * (ul % CG)) * 2;
        for (int t = 0; t < pad; t += RG)
            store16<0>(u32x4{0u, 0u, 0u, 0u}, rz, zoff + (uint32_t)(t * a.Dv * 2));
    }
}


// The segmented form's scan over an entry's segments, for one (entry, value head, 16-column
// strip). Wave w holds rows 16 w .. 16 w + 15 of the strip in fp32, in the matrix cores'
// accumulator layout: lane (g, n) = (lane / 16, lane % 16) holds rows 16 w + 4 g + i (i < 4)
// of column n. From the pool's state S, each segment j in order stores S as segment j's
// incoming state, then takes S = Phi_j S + Psi_j: Psi_j starts the accumulator, and Phi_j S
// is a 16x16x32 product per 32-row block p of S, with both operands split into bf16 high
// parts and remainders (three products, fp32 accumulation). The accumulators of waves 2 p and
// 2 p + 1 are exactly the B operand of the product over rows 32 p .. + 31 in the same lanes
// (k slots 4 g .. + 3, then 16 + 4 g .. + 3), so the waves share their split rows through
// LDS. Each segment's rows of Phi and Psi are loaded SCAN_AHEAD segments before they are
// used (rotating register sets, no copies), so the chain of segments waits on the products
// only. S is committed (bf16, round to nearest even) at the segment boundary that is the
// accepted count n: before segment ceil(n / seg_len), or after the last one.
constexpr int SCAN_AHEAD = 4;
template <int DK>
__global__ __launch_bounds__(4 * DK) void prefill_scan_kernel(
    const DecodeArgs a, const int32_t *__restrict__ lens, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nacc, const SegArgs sg) {
    constexpr int NWV = DK / 16, NKB = DK / 32;  // waves (row blocks); 32-row blocks of S
    __shared__ uint2 bfr[2][NWV][2][64];  // [segment parity][row block][hi, lo][lane]
    // The strips of one head are consecutive items, and the remap keeps consecutive items on
    // one XCD, so a head's Phi and Psi are fetched into one L2 and read there by all strips.
    const int strips = a.Dv / 16, it = xcd_item(blockIdx.x, gridDim.x);
    const int strip = it % strips, bh = it / strips;
    const int h = bh % a.Hv, b = bh / a.Hv;
    const int slot = idx[b];
    if (slot < 0 || slot >= a.N_slots) return;  // skipped entry: no state read or written
    const int L = min(max(lens[b], 0), a.T), n = min(max(nacc[b], 0), L);
    const int sl_len = sg.seg_len, na = (n + sl_len - 1) / sl_len;
    const int ns = na + (L - n + sl_len - 1) / sl_len;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nn = lane & 15, g = lane >> 4;
    const int col = strip * 16 + nn;
    const int dw = a.Dv + DK;
    const int row0 = 16 * w + 4 * g;  // this lane's state rows row0 .. row0 + 3, column col
    const size_t tbase = ((size_t)slot * a.Hv + h) * DK * a.Dv;  // the (slot, head) state
    const uint32_t lofs = (uint32_t)(row0 * a.Dv + col);          // this lane's first element
    f32x4 st;
#pragma unroll
    for (int i = 0; i < 4; ++i) st[i] = bf16_to_f32(a.pool[tbase + lofs + (size_t)i * a.Dv]);
    // One segment's operands for this lane: A fragments of Phi_j (row 16 w + nn; k slots of
    // 32-row block p: 32 p + 4 g .. + 3 and 32 p + 16 + 4 g .. + 3) and Psi_j at the state rows.
    struct Seg {
        f32x4 ph[NKB][2];
        f32x4 ps;
    };
    auto load_seg = [&](Seg &o, int j) {
        // Unconditional (a segment past the last re-reads the last allocated one, unused),
        // so that the wait counts stay static.
        j = min(j, sg.nseg - 1);
        const float *e = sg.ws_e + ((size_t)bh * sg.nseg + j) * DK * dw;
        const float *prow = e + (size_t)(16 * w + nn) * dw + a.Dv;
#pragma unroll
        for (int p = 0; p < NKB; ++p) {
            o.ph[p][0] = *reinterpret_cast<const f32x4 *>(prow + 32 * p + 4 * g);
            o.ph[p][1] = *reinterpret_cast<const f32x4 *>(prow + 32 * p + 16 + 4 * g);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) o.ps[i] = e[(size_t)(row0 + i) * dw + col];
    };
    // Segment j with its operands o; then o takes segment j + SCAN_AHEAD. Returns false
    // once every segment is done.
    auto step = [&](Seg &o, int j) {
        {
            // The state after the accepted prefix, stored at j == na (otherwise an empty
            // range drops the stores, which keeps the wait counts static).
            // (the descriptor is uniform; the lane's offset travels in the vector operand)
            const auto rc = make_rsrc(a.pool_out + tbase, j == na ? (uint32_t)(DK * a.Dv * 2) : 0u);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(st[i]), rc,
                                                      (lofs + (uint32_t)(i * a.Dv)) * 2, 0, 0);
        }
        if (j >= ns) return false;
        float *sin = sg.ws_s + ((size_t)bh * sg.nseg + j) * DK * a.Dv + (size_t)row0 * a.Dv + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) sin[(size_t)i * a.Dv] = st[i];
        {
            uint2 hi, lo;
            split4(st, hi, lo);
            bfr[j & 1][w][0][lane] = hi;
            bfr[j & 1][w][1][lane] = lo;
        }
        lds_barrier();  // (LDS only: later segments' loads stay in flight)
        f32x4 acc = o.ps;
#pragma unroll
        for (int p = 0; p < NKB; ++p) {
            const bf16x8 bh8 = cat8(bfr[j & 1][2 * p][0][lane], bfr[j & 1][2 * p + 1][0][lane]);
            const bf16x8 bl8 = cat8(bfr[j & 1][2 * p][1][lane], bfr[j & 1][2 * p + 1][1][lane]);
            uint2 ah0, al0, ah1, al1;
            split4(o.ph[p][0], ah0, al0);
            split4(o.ph[p][1], ah1, al1);
            const bf16x8 ah = cat8(ah0, ah1), al = cat8(al0, al1);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh8, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh8, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl8, acc, 0, 0, 0);
        }
        st = acc;
        load_seg(o, j + SCAN_AHEAD);
        return true;
    };
    static_assert(SCAN_AHEAD == 4, "four rotating operand sets");
    Seg s0, s1, s2, s3;
    load_seg(s0, 0);
    load_seg(s1, 1);
    load_seg(s2, 2);
    load_seg(s3, 3);
    // The parity buffers of bfr alternate by segment; a segment's writes reach the buffer the
    // segment before last read only after every wave passed the last segment's barrier.
    for (int j = 0;; j += SCAN_AHEAD) {
        if (!step(s0, j) || !step(s1, j + 1) || !step(s2, j + 2) || !step(s3, j + 3)) break;
    }
}

// One launch of n_items items, times nseg segments in the segmented passes.
template <int DK, int GATE, int NC, int SEG = 0>
static hipError_t launch_prefill(const DecodeArgs &a, const int32_t *lens, const int32_t *idx,
                                 const int32_t *nacc, const SegArgs &sg, hipStream_t stream) {
    const dim3 grid((unsigned)a.n_items * (SEG ? (unsigned)sg.nseg : 1u));
    if constexpr (GATE != kGateGiven) {
        if (a.norm_qk) {
            hipLaunchKernelGGL((prefill_kernel<DK, GATE, true, NC, SEG>), grid, dim3(256), 0,
                               stream, a, lens, idx, nacc, sg);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((prefill_kernel<DK, GATE, false, NC, SEG>), grid, dim3(256), 0, stream,
                       a, lens, idx, nacc, sg);
    return hipGetLastError();
}

template <int DK, int NC, int SEG = 0>
static hipError_t launch_prefill_gate(int gate, const DecodeArgs &a, const int32_t *lens,
                                      const int32_t *idx, const int32_t *nacc,
                                      hipStream_t stream, const SegArgs &sg = SegArgs{}) {
    return gate == kGateGiven
               ? launch_prefill<DK, kGateGiven, NC, SEG>(a, lens, idx, nacc, sg, stream)
           : gate == kGateF32 ? launch_prefill<DK, kGateF32, NC, SEG>(a, lens, idx, nacc, sg, stream)
                              : launch_prefill<DK, kGateF16, NC, SEG>(a, lens, idx, nacc, sg, stream);
}

// Compute units of the current device, queried once per device; 0 if the query fails.
static int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        return 0;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Items of the D_k = 64 kernel with 128-column tiles that the current device holds at once
// (compute units times workgroups per compute unit), queried once per device; 0 if the
// query fails.
static int prefill_resident_items_dk64() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, prefill_kernel<64, kGateGiven, false, 2>, 256, 0) != hipSuccess ||
        per_cu <= 0)
        return 0;
    n = cus * per_cu;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// The segmented form: segments per entry and their length, and the workspace they take.
// It pays where a call leaves most of the device idle: the single pass then runs at one
// item's chain of chunks, while the segmented passes run every segment at once and do about
// three times the chunk work (twice in the first pass, which carries Phi's D_k columns beside
// the D_v of Psi, once in the second). The segments are sized so that the second pass fills
// one round of two items per compute unit, and the form is taken from kSegMin of them
// (measured at T = 4096, D = 128: 8 segments 478 against 669 us in one pass; 7 segments
// were 5% slower than the single pass, 6 segments 12% faster).
constexpr int kSegMin = 8, kSegMax = 16, kSegMinLen = 64;
struct SegPlan {
    int nseg = 0, seg_len = 0;  // segments allocated per (entry, head); tokens per segment
    size_t off_s = 0, bytes = 0;  // incoming states at off_s; workspace bytes
};
static bool seg_plan(long long B, long long H_v, int T, int D_k, int D_v, int cus, SegPlan &p) {
    const long long per = B * H_v * ((D_v + 127) / 128);  // second-pass items per segment
    if (cus <= 0 || per <= 0) return false;
    const long long fit = 2LL * cus / per;
    const int want = (int)(fit < kSegMax ? fit : kSegMax);
    if (want < kSegMin) return false;
    int sl = (T + want - 1) / want;
    sl = (sl + kChunk - 1) / kChunk * kChunk;
    if (sl < kSegMinLen) return false;
    p.seg_len = sl;
    p.nseg = (T + sl - 1) / sl + 1;  // the accepted count may split one segment in two
    const size_t rows = (size_t)B * H_v * p.nseg * D_k;
    p.off_s = (rows * (D_v + D_k) * 4 + 255) / 256 * 256;
    p.bytes = p.off_s + rows * D_v * 4;
    return true;
}

template <int DK>
static hipError_t launch_segmented(DecodeArgs &a, int gate, long long B, const SegPlan &p,
                                   const int32_t *lens, const int32_t *idx, const int32_t *nacc,
                                   void *ws, hipStream_t stream) {
    SegArgs sg;
    sg.ws_e = static_cast<float *>(ws);
    sg.ws_s = reinterpret_cast<float *>(static_cast<char *>(ws) + p.off_s);
    sg.nseg = p.nseg;
    sg.seg_len = p.seg_len;
    a.item0 = 0;
    // first pass: each segment's [Psi | Phi], D_v + D_k columns in 128-column tiles
    a.ntiles = (a.Dv + DK + 127) / 128;
    a.n_items = (int)(B * a.Hv * a.ntiles);
    hipError_t err = launch_prefill_gate<DK, 2, 1>(gate, a, lens, idx, nacc, stream, sg);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((prefill_scan_kernel<DK>), dim3((unsigned)(B * a.Hv * (a.Dv / 16))),
                       dim3(4 * DK), 0, stream, a, lens, idx, nacc, sg);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    // second pass: each segment from its incoming state, the outputs
    a.ntiles = (a.Dv + 127) / 128;
    a.n_items = (int)(B * a.Hv * a.ntiles);
    return launch_prefill_gate<DK, 2, 2>(gate, a, lens, idx, nacc, stream, sg);
}

static rgdr_status prefill_entry(DecodeArgs &a, int gate, int32_t B, int32_t H_q, int32_t H_v,
                                 int32_t T, int32_t D_k, int32_t D_v, int32_t N_slots,
                                 const int32_t *lens, const int32_t *idx, const int32_t *nacc,
                                 void *ws, size_t ws_bytes, hipStream_t stream) {
    if (B < 0 || H_q <= 0 || H_v <= 0 || T <= 0 || D_k <= 0 || D_v <= 0 || N_slots <= 0)
        return RGDR_ERR_SHAPE;
    if (T > kPrefillMaxT || H_v % H_q != 0) return RGDR_ERR_SHAPE;
    // The fused gate reads [B, T, H_v] rows through one 32-bit range per entry.
    if ((long long)T * H_v > (1LL << 29)) return RGDR_ERR_SHAPE;
    if ((D_k != 64 && D_k != 128) || D_v % 64 != 0 || D_v > 4096) return RGDR_ERR_UNSUPPORTED;
    if (!aligned(a.v, 16) || !aligned(a.pool, 16) || !aligned(a.out, 16) ||
        !aligned(a.pool_out, 16) || !aligned(a.q, 16) || !aligned(a.k, 16) ||
        !aligned(a.gk, 16) || !aligned(lens, 4) || !aligned(idx, 4) || !aligned(nacc, 4))
        return RGDR_ERR_ALIGN;
    if (ws != nullptr) {  // the segmented form, where it pays and the workspace holds it
        const int cus = device_cus();
        if (cus <= 0) return RGDR_ERR_HIP;
        SegPlan p;
        if (seg_plan(B, H_v, T, D_k, D_v, cus, p) && ws_bytes >= p.bytes && aligned(ws, 256)) {
            a.Hq = H_q;
            a.Hv = H_v;
            a.T = T;
            a.Dv = D_v;
            a.N_slots = N_slots;
            a.group = H_v / H_q;
            const hipError_t err =
                D_k == 128 ? launch_segmented<128>(a, gate, B, p, lens, idx, nacc, ws, stream)
                           : launch_segmented<64>(a, gate, B, p, lens, idx, nacc, ws, stream);
            return err == hipSuccess ? RGDR_OK : RGDR_ERR_HIP;
        }
    }
    // Tiles of 128 columns (the last may be 64 wide). At D_k = 64, 256-column tiles (D_v a
    // multiple of 256) when the call has more 128-column items than the device holds at once:
    // half as many items, each with the state bytes of a D_k = 128 item, so fewer rounds of
    // items pay the per-chunk work that does not scale with the columns.
    // At D_k = 128, 64-column tiles when the call has at most half as many 128-column items
    // as the device has compute units. Such a call runs at one item's chain of chunks, and
    // the chain is bound by its compute unit's issue of the column work (the contraction
    // with the state, the update, the state's split). Twice the items, each with half the
    // columns and still one per unit, shorten it; the per-token preparation is repeated.
    int tile_v = 128;
    bool narrow = false;
    if (D_k == 64 && D_v % 256 == 0) {
        const int resident = prefill_resident_items_dk64();
        if (resident <= 0) return RGDR_ERR_HIP;
        if ((long long)B * H_v * (D_v / 128) > resident) tile_v = 256;
    } else if (D_k == 128) {
        const int cus = device_cus();
        if (cus <= 0) return RGDR_ERR_HIP;
        if (2LL * B * H_v * ((D_v + 127) / 128) <= cus) {
            narrow = true;
            tile_v = 64;
        }
    }
    const int ntiles = (D_v + tile_v - 1) / tile_v;
    const long long items = (long long)B * H_v * ntiles;
    if (items > INT_MAX) return RGDR_ERR_SHAPE;
    a.Hq = H_q;
    a.Hv = H_v;
    a.T = T;
    a.Dv = D_v;
    a.N_slots = N_slots;
    a.ntiles = ntiles;
    a.group = H_v / H_q;
    a.n_items = (int)items;
    a.item0 = 0;
    hipError_t err;
    if (D_k == 128 && narrow)
        err = launch_prefill_gate<128, 1>(gate, a, lens, idx, nacc, stream);
    else if (D_k == 128)
        err = launch_prefill_gate<128, 2>(gate, a, lens, idx, nacc, stream);
    else if (tile_v == 256)
        err = launch_prefill_gate<64, 4>(gate, a, lens, idx, nacc, stream);
    else
        err = launch_prefill_gate<64, 2>(gate, a, lens, idx, nacc, stream);
    return err == hipSuccess ? RGDR_OK : RGDR_ERR_HIP;
}

static rgdr_status prefill_given(const void *query, const void *key, const void *value,
                                 const void *beta, const void *state_pool, const int32_t *lens,
                                 const int32_t *idx, const float *g, const float *gk,
                                 const int32_t *nacc, float scale, int32_t B, int32_t H_q,
                                 int32_t H_v, int32_t T, int32_t D_k, int32_t D_v,
                                 int32_t N_slots, void *out, void *state_out, void *ws,
                                 size_t ws_bytes, hipStream_t stream) {
    if (B == 0) return RGDR_OK;
    if (!query || !key || !value || !beta || !state_pool || !lens || !idx || !g || !gk ||
        !nacc || !out || !state_out)
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
    return prefill_entry(a, kGateGiven, B, H_q, H_v, T, D_k, D_v, N_slots, lens, idx, nacc, ws,
                         ws_bytes, stream);
}

static rgdr_status prefill_gated(const void *query, const void *key, const void *value,
                                 const void *gate_a, const void *gate_b, const float *dt_bias,
                                 const float *decay_scale, rgdr_dtype gate_dtype,
                                 const void *state_pool, const int32_t *lens,
                                 const int32_t *idx, const float *gk, const int32_t *nacc,
                                 float scale, int32_t B, int32_t H_q, int32_t H_v, int32_t T,
                                 int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
                                 void *state_out, uint32_t flags, void *ws, size_t ws_bytes,
                                 hipStream_t stream) {
    if (flags & ~(uint32_t)RGDR_NORMALIZE_QK) return RGDR_ERR_UNSUPPORTED;
    if (B == 0) return RGDR_OK;
    if (!query || !key || !value || !gate_a || !gate_b || !dt_bias || !decay_scale ||
        !state_pool || !lens || !idx || !gk || !nacc || !out || !state_out)
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
    a.scale = scale;
    return prefill_entry(a, gate_dtype == RGDR_F16 ? kGateF16 : kGateF32, B, H_q, H_v, T, D_k,
                         D_v, N_slots, lens, idx, nacc, ws, ws_bytes, stream);
}

// Allocation-free form of rgdr_prefill_ws: the segmented form's workspace is this file-scope
// device array, held by every device the library runs on until the process ends. Host code
// never passes the array's name to a kernel (on the host it is a stand-in, not a device
// address): each device's address is looked up once, with that device current.
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

static rgdr_status scratch_address(void **out) {
    static std::atomic<void *> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return RGDR_ERR_HIP;
    void *p = cached[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return RGDR_ERR_HIP;
        cached[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return RGDR_OK;
}

}  // namespace rgdr

extern "C" rgdr_status rgdr_prefill(const void *query, const void *key, const void *value,
                                    const void *beta, const void *state_pool,
                                    const int32_t *actual_seq_lengths,
                                    const int32_t *ssm_state_indices, const float *g,
                                    const float *gk, const int32_t *num_accepted_tokens,
                                    float scale, int32_t B, int32_t H_q, int32_t H_v,
                                    int32_t T, int32_t D_k, int32_t D_v, int32_t N_slots,
                                    void *out, void *state_out, hipStream_t stream) {
    return rgdr::prefill_given(query, key, value, beta, state_pool, actual_seq_lengths,
                               ssm_state_indices, g, gk, num_accepted_tokens, scale, B, H_q,
                               H_v, T, D_k, D_v, N_slots, out, state_out, nullptr, 0, stream);
}

extern "C" rgdr_status rgdr_prefill_gated(
    const void *query, const void *key, const void *value, const void *gate_a,
    const void *gate_b, const float *dt_bias, const float *decay_scale, rgdr_dtype gate_dtype,
    const void *state_pool, const int32_t *actual_seq_lengths, const int32_t *ssm_state_indices,
    const float *gk, const int32_t *num_accepted_tokens, float scale, int32_t B, int32_t H_q,
    int32_t H_v, int32_t T, int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
    void *state_out, uint32_t flags, hipStream_t stream) {
    return rgdr::prefill_gated(query, key, value, gate_a, gate_b, dt_bias, decay_scale,
                               gate_dtype, state_pool, actual_seq_lengths, ssm_state_indices, gk,
                               num_accepted_tokens, scale, B, H_q, H_v, T, D_k, D_v, N_slots,
                               out, state_out, flags, nullptr, 0, stream);
}

extern "C" rgdr_status rgdr_prefill_workspace_size(int32_t B, int32_t H_v, int32_t T,
                                                   int32_t D_k, int32_t D_v, size_t *bytes) {
    using namespace rgdr;
    if (!bytes) return RGDR_ERR_NULL;
    *bytes = 0;
    if (B < 0 || H_v <= 0 || T <= 0 || D_k <= 0 || D_v <= 0 || T > kPrefillMaxT)
        return RGDR_ERR_SHAPE;
    if ((D_k != 64 && D_k != 128) || D_v % 64 != 0 || D_v > 4096) return RGDR_ERR_UNSUPPORTED;
    if (B == 0) return RGDR_OK;
    const int cus = device_cus();
    if (cus <= 0) return RGDR_ERR_HIP;
    SegPlan p;
    if (seg_plan(B, H_v, T, D_k, D_v, cus, p)) *bytes = p.bytes;
    return RGDR_OK;
}

extern "C" rgdr_status rgdr_prefill_ws(const void *query, const void *key, const void *value,
                                       const void *beta, const void *state_pool,
                                       const int32_t *actual_seq_lengths,
                                       const int32_t *ssm_state_indices, const float *g,
                                       const float *gk, const int32_t *num_accepted_tokens,
                                       float scale, int32_t B, int32_t H_q, int32_t H_v,
                                       int32_t T, int32_t D_k, int32_t D_v, int32_t N_slots,
                                       void *out, void *state_out, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    return rgdr::prefill_given(query, key, value, beta, state_pool, actual_seq_lengths,
                               ssm_state_indices, g, gk, num_accepted_tokens, scale, B, H_q,
                               H_v, T, D_k, D_v, N_slots, out, state_out, workspace,
                               workspace_bytes, stream);
}

extern "C" rgdr_status rgdr_prefill_gated_ws(
    const void *query, const void *key, const void *value, const void *gate_a,
    const void *gate_b, const float *dt_bias, const float *decay_scale, rgdr_dtype gate_dtype,
    const void *state_pool, const int32_t *actual_seq_lengths, const int32_t *ssm_state_indices,
    const float *gk, const int32_t *num_accepted_tokens, float scale, int32_t B, int32_t H_q,
    int32_t H_v, int32_t T, int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
    void *state_out, uint32_t flags, void *workspace, size_t workspace_bytes,
    hipStream_t stream) {
    return rgdr::prefill_gated(query, key, value, gate_a, gate_b, dt_bias, decay_scale,
                               gate_dtype, state_pool, actual_seq_lengths, ssm_state_indices, gk,
                               num_accepted_tokens, scale, B, H_q, H_v, T, D_k, D_v, N_slots,
                               out, state_out, flags, workspace, workspace_bytes, stream);
}

extern "C" rgdr_status rgdr_prefill_noalloc(const void *query, const void *key,
                                            const void *value, const void *beta,
                                            const void *state_pool,
                                            const int32_t *actual_seq_lengths,
                                            const int32_t *ssm_state_indices, const float *g,
                                            const float *gk,
                                            const int32_t *num_accepted_tokens, float scale,
                                            int32_t B, int32_t H_q, int32_t H_v, int32_t T,
                                            int32_t D_k, int32_t D_v, int32_t N_slots,
                                            void *out, void *state_out, hipStream_t stream) {
    using namespace rgdr;
    size_t need = 0;
    if (B > 0 && H_q > 0 && H_v > 0 && T > 0 && T <= kPrefillMaxT && (D_k == 64 || D_k == 128) &&
        D_v > 0 && D_v % 64 == 0 && D_v <= 4096) {
        // sizes the other checks refuse fall through to them below
        const rgdr_status st = rgdr_prefill_workspace_size(B, H_v, T, D_k, D_v, &need);
        if (st != RGDR_OK) return st;
        if (need > kScratchBytes) return RGDR_ERR_SCRATCH;
    }
    void *ws = nullptr;
    if (need > 0) {
        const rgdr_status st = scratch_address(&ws);
        if (st != RGDR_OK) return st;
    }
    return prefill_given(query, key, value, beta, state_pool, actual_seq_lengths,
                         ssm_state_indices, g, gk, num_accepted_tokens, scale, B, H_q, H_v, T,
                         D_k, D_v, N_slots, out, state_out, ws, ws ? kScratchBytes : 0, stream);
}
