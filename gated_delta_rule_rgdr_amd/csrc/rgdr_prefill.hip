// rgdr_prefill.hip -- the gated-delta recurrence over long sequences (T > 8) on gfx950.
//
// Method: MindSpore Lite API page "lite_boost.ops.recurrent_gated_delta_rule". Its
// algorithm section gives the four steps applied token by token; its notes limit that
// decode operator to T <= 8 and send the parallel prefill to a chunk-level operator. This
// is that operator for this library: the same inputs, outputs and semantics as rgdr_decode
// (slot pool, lengths, accepted counts, head sharing, padding), for any T up to 65536.
//
// Design. One workgroup of two waves owns one (entry, value head, 128-column tile) for the
// whole sequence. Its state tile is read from HBM once, kept in fp32 in the matrix cores'
// accumulator layout while the item's tokens are walked in runs of at most 8, and written
// back once (at the accepted prefix's end). Each run is the exact closed form of the decode
// kernel's chunk form (decay products c_t, the 8 x 8 matrices M and N, a triangular solve
// for u, then the committed state diag(c) S + (g k)^T U), with S the running fp32 state:
//   * Y = [c k | c scale q]^T S on the matrix cores, S split into a bf16 high part and a
//     bf16 remainder (exact in fp32) against the operands' high parts and remainders, so
//     the products keep about 16 bits of every operand;
//   * the row scaling diag(c) S on the VALU, in fp32, on the accumulator registers;
//   * the rank-8 update (g k)^T U as matrix-core products accumulating into S.
// The run that holds the accepted prefix's end stops there, so the committed state is a
// run's end state; the later tokens still produce their outputs. The next run's operands
// are loaded while the current run is computed. HBM sees the state once in and once out,
// and every operand once.
#include <climits>

#include "rgdr_device.h"

namespace rgdr {

constexpr int kPrefillMaxT = 65536;  // tokens per call: keeps every per-item offset in 32 bits

// Waves per SIMD the kernel is compiled for (the register budget).
#ifndef RGDR_PREFILL_MIN_WAVES
#define RGDR_PREFILL_MIN_WAVES 2
#endif

// f32x4 pair -> bf16 high parts and bf16 remainders, 8 values in k order (x0 first).
__device__ __forceinline__ void split8(const f32x4 &x0, const f32x4 &x1, bf16x8 &hi,
                                       bf16x8 &lo) {
    const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        // x - hi is exact in fp32
        l[j] = pack_bf16x2(v[2 * j] - bf16_lo(h[j]), v[2 * j + 1] - bf16_hi(h[j]));
    }
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

// Lane layout. Four waves per item; wave w owns tile columns 32 w .. 32 w + 31 over all D_k
// rows. Lane l = (kg, n16) = (l / 16, l % 16) holds state rows 16 rb + 4 kg + i (rb < D_k / 16,
// i < 4) of columns 32 w + 2 n16 + c (c < 2) as S[rb][c][i]: the accumulator layout of the
// 16 x 16 block of rows 16 rb .. + 15 and columns 32 w + 2 n + c (column set c). Rows
// 4 kg .. 4 kg + 3 of two row blocks are also the 8 k slots of lane group kg in a 16x16x32
// product, so the state turns into the B operand of Y = X^T S in the lane that holds it.
// At 64 state values per lane two waves fit a SIMD.
template <int DK, int GATE>
__global__ __launch_bounds__(256, RGDR_PREFILL_MIN_WAVES) void prefill_kernel(
    const DecodeArgs a, const int32_t *__restrict__ lens, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nacc) {
    static_assert(DK == 64 || DK == 128, "D_k = 64 or 128");
    constexpr int TV = 128, NT = 256, NW = 4;
    constexpr int NRB = DK / 16, NPB = DK / 32;
    // LDS: staged operands of one run (chunk_stage_ops) | XT hi, lo [16][XS] (c k | c scale
    // q) | KC hi, lo [8][XS] (k_s / c_s) | KA hi, lo [D_k][8] | UT
    // [wave][hi, lo][2 column sets][16][8] | c of each row at the run's end [D_k] | direct
    // Gram partials [2][64] | M and N [wave][8][8]. Y^T [128][kChunkYS] takes the d, k and q
    // planes once the rows are prepared.
    constexpr int XS = DK + 4;
    constexpr int VB = chunk_vbase<DK>();
    constexpr int OFF_XT = chunk_ops<DK>() * 4;
    constexpr int OFF_KC = OFF_XT + 2 * 16 * XS * 2;
    constexpr int OFF_KA = OFF_KC + 2 * 8 * XS * 2;
    constexpr int OFF_UT = OFF_KA + 2 * DK * 8 * 2;
    constexpr int OFF_CL = OFF_UT + NW * 2 * 2 * 16 * 8 * 2;
    constexpr int OFF_GP = OFF_CL + DK * 4;
    constexpr int OFF_GS = OFF_GP + 2 * 64 * 4;
    constexpr int BYTES = OFF_GS + NW * 2 * 64 * 4;
    static_assert(BYTES % 16 == 0 && BYTES <= 81920, "LDS carve: two items per compute unit");
    constexpr int YS = kChunkYS;
    __shared__ f32x4 lds4[BYTES / 16];
    char *lb = reinterpret_cast<char *>(lds4);
    float *ob = reinterpret_cast<float *>(lb);
    uint16_t *xt_hi = reinterpret_cast<uint16_t *>(lb + OFF_XT), *xt_lo = xt_hi + 16 * XS;
    uint16_t *kc_hi = reinterpret_cast<uint16_t *>(lb + OFF_KC), *kc_lo = kc_hi + 8 * XS;
    uint16_t *ka_hi = reinterpret_cast<uint16_t *>(lb + OFF_KA), *ka_lo = ka_hi + DK * 8;
    float *crow = reinterpret_cast<float *>(lb + OFF_CL);
    float *gpart = reinterpret_cast<float *>(lb + OFF_GP);

    const Index x{lens, idx, nacc};
    const int tid = threadIdx.x, lane = tid & 63, n16 = lane & 15, kg = lane >> 4;
    // w is the same in every lane of a wave; readfirstlane tells the compiler so, which keeps
    // the buffer descriptors built from it in scalar registers.
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint16_t *ut_hi = reinterpret_cast<uint16_t *>(lb + OFF_UT) + w * 2 * 32 * 8, *ut_lo = ut_hi + 32 * 8;
    float *gsM = reinterpret_cast<float *>(lb + OFF_GS) + w * 2 * 64, *gsN = gsM + 64;
    const Item m = resolve(a, x, xcd_item(blockIdx.x, gridDim.x));
    const int L = m.L, n = m.n;
    auto ycol = [&](int j) { return ob + j * YS; };

    // A last tile of 64 columns (D_v an odd multiple of 64) leaves waves 2 and 3 without
    // columns: their state and output accesses get empty ranges and they compute on zeros.
    const bool cols = m.tile * TV + 32 * w < a.Dv;
    const uint32_t trange = cols ? tile_range<DK, TV>(a, m) : 0u;
    const size_t tb = m.state ? tile_base<DK, TV>(a, m) : 0;
    const auto rs = make_rsrc(a.pool + tb, trange);
    const auto rso = make_rsrc(a.pool_out + tb, trange);
    const uint32_t lane_off = (uint32_t)((4 * kg * a.Dv + 32 * w + 2 * n16) * 2);
    const size_t bh = (size_t)m.b * a.Hv + m.h;
    const int jcol = lane & 31;       // this lane's local column in the solve
    const int col = 32 * w + jcol;    // lanes 32..63 repeat lanes 0..31 and store nothing
    const uint32_t ocol = lane < 32 ? (uint32_t)((m.tile * TV + col) * 2) : 0x40000000u;

    // Runs of at most kMaxT tokens; the run holding the accepted prefix's end stops there.
    auto run_end = [&](int t0) {
        const int t1 = min(t0 + kMaxT, L);
        return (t0 < n && n < t1) ? n : t1;
    };

    // The first run's operands, then the state tile (bf16 -> fp32, exact).
    int t0 = 0, t1 = run_end(0);
    Ops<DK, TV, NT, kMaxT> o;
    load_ops<DK, TV, NT, kMaxT, GATE>(a, m, o, tid, 0, t1);
    uint32_t raw[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            raw[rb][i] = __builtin_amdgcn_raw_buffer_load_b32(
                rs, lane_off, (uint32_t)((16 * rb + i) * a.Dv * 2), RGDR_STATE_LOAD_POLICY);
    f32x4 S[NRB][2];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            S[rb][0][i] = bf16_lo(raw[rb][i]);
            S[rb][1][i] = bf16_hi(raw[rb][i]);
        }
    if (n == 0) {  // nothing accepted: commit the incoming bytes
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(
                    raw[rb][i], rso, lane_off + (uint32_t)((16 * rb + i) * a.Dv * 2), 0,
                    RGDR_STATE_STORE_POLICY);
    }

    while (t0 < L) {  // uniform over the workgroup
        const int Lc = t1 - t0;
        chunk_stage_ops<DK, GATE, NT>(o, ob, a.scale, a.norm_qk != 0, Lc, tid);
        // The next run's operands travel while this run is computed (zeros past the end).
        const int t0n = t1, t1n = t1 < L ? run_end(t1) : t1;
        __builtin_amdgcn_sched_barrier(0);
        load_ops<DK, TV, NT, kMaxT, GATE>(a, m, o, tid, t0n, t1n - t0n);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();

        // Per-row preparation: thread r owns row r (waves 0 and 1 at D_k = 128, wave 0 at
        // D_k = 64).
        const bool has_rows = 64 * w < DK;
        bool direct = false;  // this wave forms its rows' Gram shares directly
        float gp[64];  // direct partial G: [t][s] (s <= t) holds N[t][s], [s][t] (s < t) M[t][s]
#pragma unroll
        for (int e = 0; e < 64; ++e) gp[e] = 0.f;
        if (has_rows) {
            const int row = tid;
            float d[8], k[8], q[8], c[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                d[t] = ob[t * DK + row];  // tokens past the run were staged neutral (d = 1)
                k[t] = ob[8 * DK + t * DK + row];
                q[t] = ob[16 * DK + t * DK + row];
            }
            float cc = 1.f, cend = 1.f, cmin = 1.f, cmax = 1.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                cc *= d[t];
                c[t] = cc;
                cmin = fminf(cmin, cc);
                cmax = fmaxf(cmax, cc);
                uint16_t hk, lk, hq, lq;
                split_bf16(cc * k[t], hk, lk);
                split_bf16(cc * q[t], hq, lq);
                xt_hi[t * XS + row] = hk;
                xt_lo[t * XS + row] = lk;
                xt_hi[(8 + t) * XS + row] = hq;
                xt_lo[(8 + t) * XS + row] = lq;
                if (t + 1 == Lc) cend = cc;
            }
            crow[row] = cend;
            direct = __ballot(!(cmin >= kGramLo && cmax <= kGramHi)) != 0;  // NaN: direct
            float ka[8];
            if (!direct) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float kcs = k[s] * __builtin_amdgcn_rcpf(c[s]);  // k_s / c_s
                    uint16_t h, l;
                    split_bf16(kcs, h, l);
                    kc_hi[s * XS + row] = h;
                    kc_lo[s * XS + row] = l;
                    ka[s] = s < Lc ? cend * kcs : 0.f;  // g(Lc-1, s) k_s
                }
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    kc_hi[s * XS + row] = 0;
                    kc_lo[s * XS + row] = 0;
                    float wv = k[s];  // g(s,s) k_s
                    ka[s] = (s + 1 == Lc) ? wv : 0.f;
                    gp[s * 8 + s] = wv * q[s];
#pragma unroll
                    for (int t = s + 1; t < 8; ++t) {
                        wv *= d[t];  // g(t,s) k_s
                        gp[s * 8 + t] = wv * k[t];
                        gp[t * 8 + s] = wv * q[t];
                        if (t + 1 == Lc) ka[s] = wv;
                    }
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
        if (w < 2)  // the direct shares of this wave's rows (zero where none): lane e, entry e
            gpart[64 * w + lane] = direct ? wave_sum64_transposed(gp, lane) : 0.f;
        lds_barrier();

        // M and N: the factored products on the matrix cores (each wave for itself), plus
        // the direct shares.
        gram_tables<DK, XS>(xt_hi, xt_lo, kc_hi, kc_lo, gpart, gsM, gsN, n16, kg);
        lds_phase();

        // Y = [c k | c scale q]^T S (16 x 32, this wave's columns), column set c, over
        // row-block pairs; three products of the split parts (high x high, low x high,
        // high x low).
        f32x4 acc[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
            const int r0 = 32 * pb + 4 * kg;
            const bf16x8 ah = lds_pair8(xt_hi + n16 * XS + r0, xt_hi + n16 * XS + r0 + 16);
            const bf16x8 al = lds_pair8(xt_lo + n16 * XS + r0, xt_lo + n16 * XS + r0 + 16);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                bf16x8 sh, sl;
                split8(S[2 * pb][c], S[2 * pb + 1][c], sh, sl);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sh, acc[c], 0, 0, 0);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, sh, acc[c], 0, 0, 0);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sl, acc[c], 0, 0, 0);
            }
        }
        // Y to LDS, transposed: accumulator c holds rows 4 kg .. 4 kg + 3 of column
        // 32 w + 2 n16 + c. Every wave has prepared its rows (barrier above), so the d, k and
        // q planes are free.
#pragma unroll
        for (int c = 0; c < 2; ++c)
            *reinterpret_cast<f32x4 *>(ycol(32 * w + 2 * n16 + c) + 4 * kg) = acc[c];
        lds_phase();

        // Triangular solve for column 32 w + (lane & 31); outputs of the run's tokens.
        const auto rout = make_rsrc(a.out + (bh * a.T + t0) * a.Dv,
                                    cols ? (uint32_t)(Lc * a.Dv * 2) : 0u);
        float yc[16];
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const f32x4 e = *reinterpret_cast<const f32x4 *>(ycol(col) + 4 * v4);
            yc[4 * v4] = e.x;
            yc[4 * v4 + 1] = e.y;
            yc[4 * v4 + 2] = e.z;
            yc[4 * v4 + 3] = e.w;
        }
        float u[8];
        uint16_t o16[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float v = ob[VB + t * TV + col];
            const float bt = ob[VB + 8 * TV + t];
            float p = yc[t];
#pragma unroll
            for (int s2 = 0; s2 < t; ++s2) p = fmaf(gsM[t * 8 + s2], u[s2], p);
            u[t] = t < Lc ? bt * (v - p) : 0.f;
            float ov = yc[8 + t];
#pragma unroll
            for (int s2 = 0; s2 <= t; ++s2) ov = fmaf(gsN[t * 8 + s2], u[s2], ov);
            o16[t] = f32_to_bf16(ov);
        }
        // rows past the run fall outside the output range and are not written
#pragma unroll
        for (int t = 0; t < 8; ++t)
            __builtin_amdgcn_raw_buffer_store_b16(o16[t], rout, (uint32_t)(t * a.Dv * 2) + ocol, 0, 0);
        {
            uint16_t h[8], l[8];
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) split_bf16(u[s2], h[s2], l[s2]);
            // local column j = 2 n + c goes to UT position c * 16 + n (lanes 32..63 write
            // the same values as lanes 0..31)
            const int p = (jcol & 1) * 16 + (jcol >> 1);
            *reinterpret_cast<u32x4 *>(ut_hi + p * 8) =
                u32x4{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                      h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
            *reinterpret_cast<u32x4 *>(ut_lo + p * 8) =
                u32x4{l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16),
                      l[4] | ((uint32_t)l[5] << 16), l[6] | ((uint32_t)l[7] << 16)};
        }
        lds_phase();

        // S = diag(c_end) S + [g k]^T U. The row scaling is an fp32 multiply of the
        // accumulators; the update is two 16x16x16 products per block into them: lane group kg
        // carries tokens 4 (kg & 1) .. + 3 of A's high part (kg < 2) or remainder (kg >= 2),
        // against U's high part, then U's remainder. Only this one instruction shape ever
        // accumulates into S.
        s16x4 buh[2], bul[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            buh[c] = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(ut_hi + (c * 16 + n16) * 8 + 4 * (kg & 1)));
            bul[c] = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(ut_lo + (c * 16 + n16) * 8 + 4 * (kg & 1)));
        }
        const uint16_t *ka_lane = (kg >> 1 ? ka_lo : ka_hi) + n16 * 8 + 4 * (kg & 1);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const f32x4 cr = *reinterpret_cast<const f32x4 *>(crow + 16 * rb + 4 * kg);
            const s16x4 ak = __builtin_bit_cast(s16x4, *reinterpret_cast<const uint2 *>(ka_lane + 16 * rb * 8));
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                S[rb][c] = S[rb][c] * cr;
                S[rb][c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ak, buh[c], S[rb][c], 0, 0, 0);
                S[rb][c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ak, bul[c], S[rb][c], 0, 0, 0);
            }
        }
        t0 = t1;
        t1 = t1n;
        if (t0 == n) {  // the accepted prefix ends here: commit
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        pack_bf16x2(S[rb][0][i], S[rb][1][i]), rso,
                        lane_off + (uint32_t)((16 * rb + i) * a.Dv * 2), 0,
                        RGDR_STATE_STORE_POLICY);
        }
        lds_barrier();  // the next run's staging reuses every LDS area
    }

    // Padded (or skipped) tokens: +0.0 rows. Lane (r, c4) stores 8 columns of row r of each
    // group of 16 rows; rows past T fall outside the range.
    if (cols && L < a.T) {
        const int pad = a.T - L;
        const auto rz = make_rsrc(a.out + (bh * a.T + L) * a.Dv + m.tile * TV + 32 * w,
                                  (uint32_t)(((pad - 1) * a.Dv + 32) * 2));
        const uint32_t zoff = (uint32_t)(((lane >> 2) * a.Dv + 8 * (lane & 3)) * 2);
        for (int t = 0; t < pad; t += 16)
            store16<0>(u32x4{0u, 0u, 0u, 0u}, rz, zoff + (uint32_t)(t * a.Dv * 2));
    }
}

template <int DK, int GATE>
static hipError_t launch_prefill(const DecodeArgs &a, const int32_t *lens, const int32_t *idx,
                                 const int32_t *nacc, hipStream_t stream) {
    hipLaunchKernelGGL((prefill_kernel<DK, GATE>), dim3(a.n_items), dim3(256), 0, stream, a,
                       lens, idx, nacc);
    return hipGetLastError();
}

static rgdr_status prefill_entry(DecodeArgs &a, int gate, int32_t B, int32_t H_q, int32_t H_v,
                                 int32_t T, int32_t D_k, int32_t D_v, int32_t N_slots,
                                 const int32_t *lens, const int32_t *idx, const int32_t *nacc,
                                 hipStream_t stream) {
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
    const int ntiles = (D_v + 127) / 128;  // the last tile may be 64 columns wide
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
    if (D_k == 128)
        err = gate == kGateGiven ? launch_prefill<128, kGateGiven>(a, lens, idx, nacc, stream)
              : gate == kGateF32 ? launch_prefill<128, kGateF32>(a, lens, idx, nacc, stream)
                                 : launch_prefill<128, kGateF16>(a, lens, idx, nacc, stream);
    else
        err = gate == kGateGiven ? launch_prefill<64, kGateGiven>(a, lens, idx, nacc, stream)
              : gate == kGateF32 ? launch_prefill<64, kGateF32>(a, lens, idx, nacc, stream)
                                 : launch_prefill<64, kGateF16>(a, lens, idx, nacc, stream);
    return err == hipSuccess ? RGDR_OK : RGDR_ERR_HIP;
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
    using namespace rgdr;
    if (B == 0) return RGDR_OK;
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
    return prefill_entry(a, kGateGiven, B, H_q, H_v, T, D_k, D_v, N_slots, actual_seq_lengths,
                         ssm_state_indices, num_accepted_tokens, stream);
}

extern "C" rgdr_status rgdr_prefill_gated(
    const void *query, const void *key, const void *value, const void *gate_a,
    const void *gate_b, const float *dt_bias, const float *decay_scale, rgdr_dtype gate_dtype,
    const void *state_pool, const int32_t *actual_seq_lengths, const int32_t *ssm_state_indices,
    const float *gk, const int32_t *num_accepted_tokens, float scale, int32_t B, int32_t H_q,
    int32_t H_v, int32_t T, int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
    void *state_out, uint32_t flags, hipStream_t stream) {
    using namespace rgdr;
    if (flags & ~(uint32_t)RGDR_NORMALIZE_QK) return RGDR_ERR_UNSUPPORTED;
    if (B == 0) return RGDR_OK;
    if (!query || !key || !value || !gate_a || !gate_b || !dt_bias || !decay_scale ||
        !state_pool || !actual_seq_lengths || !ssm_state_indices || !gk ||
        !num_accepted_tokens || !out || !state_out)
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
                         D_v, N_slots, actual_seq_lengths, ssm_state_indices,
                         num_accepted_tokens, stream);
}
