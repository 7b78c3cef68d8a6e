// rgdr_decode.hip -- the recurrent gated-delta-rule decode step on gfx950 (MI355X).
//
// Method: MindSpore Lite API page "lite_boost.ops.recurrent_gated_delta_rule", algorithm
// section (decay, memory read, delta update, output, token by token) and parameter list.
//
// The step is HBM-bound: each (batch entry, value head) pair streams its D_k x D_v bf16
// state in once and out once, and everything else is small. One workgroup owns one
// (b, h, D_v tile) and keeps that tile in fp32 registers across all tokens:
//
//   * a thread owns 8 consecutive columns (one 16-byte bf16 vector) of R rows spaced
//     RPP apart, so every load/store instruction of the workgroup covers RPP whole tile
//     rows, contiguous in memory; all state loads are issued before anything else;
//   * per-token operands (decay factors exp(g) exp(gk), k, q * scale, the v tile, beta)
//     are staged once in LDS for all tokens;
//   * per token, steps 2 and 4 share ONE reduction over D_k: with S' the decayed state,
//     p = S'^T k and r = S'^T (scale q) are reduced together with the scalar k.(scale q),
//     then u = beta (v - p), o = r + (k.(scale q)) u, which equals S_new^T (scale q), and
//     S_new = S' + k (x) u is one FMA per element;
//   * the reduction is in-thread over R rows, then a butterfly across the lanes of the
//     wave that hold the same columns, then a fixed-order sum over the waves through a
//     double-buffered LDS slot (one barrier per token). Results are deterministic.
//
// No matrix cores: the work per token is a matrix-vector product and a rank-1 update.
#include "rgdr_common.h"

namespace rgdr {

constexpr int kMaxT = 8;  // decode only: at most 8 tokens per call

struct DecodeArgs {
    const uint16_t *q, *k, *v, *beta, *pool;
    const int32_t *lens, *idx, *nacc;
    const float *g, *gk;
    uint16_t *out, *pool_out;
    float scale;
    int Hq, Hv, T, Dv, N_slots, ntiles, group;
};

template <int DK, int TV, int NT>
struct TileShape {
    static constexpr int CPL = 8;         // columns per lane: one 16-byte bf16 vector
    static constexpr int LPR = TV / CPL;  // lanes across one tile row
    static constexpr int RPP = NT / LPR;  // tile rows covered per pass of the workgroup
    static constexpr int R = DK / RPP;    // rows held by each thread
    static constexpr int NW = NT / 64;    // waves per workgroup
    static_assert(NT % 64 == 0 && 64 % LPR == 0 && DK % RPP == 0 && R >= 1, "tile shape");
    // LDS, in floats. Per token: decay[DK] | k[DK] | scale*q[DK] | v[TV] | beta.
    static constexpr int TOK = 3 * DK + TV + 1;
    // Reduction exchange, two buffers of: per wave p[TV] | r[TV] | k.q.
    static constexpr int EXW = 2 * TV + 1;
    static constexpr int EX = NW * EXW;
    static size_t lds_bytes(int T) { return sizeof(float) * (size_t)(T * TOK + 2 * EX); }
};

template <int DK, int TV, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(const DecodeArgs a) {
    using Sh = TileShape<DK, TV, NT>;
    constexpr int CPL = Sh::CPL, LPR = Sh::LPR, RPP = Sh::RPP, R = Sh::R, NW = Sh::NW;
    extern __shared__ float lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = tid % LPR;  // column group: columns cg*8 .. cg*8+7 of the tile
    const int rg = tid / LPR;  // row group: rows rg, rg+RPP, ...

    const int tile = blockIdx.x % a.ntiles;
    const int bh = blockIdx.x / a.ntiles;  // b * H_v + h
    const int h = bh % a.Hv;
    const int b = bh / a.Hv;
    const int hq = h / a.group;  // shared query/key head, floor(h * H_q / H_v)
    const int T = a.T;

    // Index resolve: the slot, the valid length L and the committed prefix n.
    const int slot = a.idx[b];
    const bool valid = slot >= 0 && slot < a.N_slots;
    int L = min(max(a.lens[b], 0), T);
    const int n = min(max(a.nacc[b], 0), L);
    if (!valid) L = 0;  // skipped entry: zero output, no state access

    const int col0 = tile * TV + cg * CPL;
    const size_t bhT = (size_t)bh * T;
    uint16_t *out_row = a.out + bhT * a.Dv + col0;
    const size_t srow0 = ((size_t)slot * a.Hv + h) * DK;  // first state row of the pair

    // State gather: every 16-byte load of the tile is in flight before other work.
    uint4 raw[R];
    if (valid) {
        const uint16_t *src = a.pool + srow0 * a.Dv + col0;
#pragma unroll
        for (int r = 0; r < R; ++r)
            raw[r] = *reinterpret_cast<const uint4 *>(src + (size_t)(rg + r * RPP) * a.Dv);
    }

    // Operand staging for the L valid tokens.
    const size_t qk0 = ((size_t)b * a.Hq + hq) * T;
    for (int e = tid; e < L * DK; e += NT) {
        const int t = e / DK, i = e - t * DK;
        float *tok = lds + t * Sh::TOK;
        tok[i] = __expf(a.g[bhT + t]) * __expf(a.gk[(bhT + t) * DK + i]);
        tok[DK + i] = bf16_to_f32(a.k[(qk0 + t) * DK + i]);
        tok[2 * DK + i] = bf16_to_f32(a.q[(qk0 + t) * DK + i]) * a.scale;
    }
    for (int e = tid; e < L * TV; e += NT) {
        const int t = e / TV, c = e - t * TV;
        lds[t * Sh::TOK + 3 * DK + c] = bf16_to_f32(a.v[(bhT + t) * a.Dv + tile * TV + c]);
    }
    if (tid < L) lds[tid * Sh::TOK + 3 * DK + TV] = bf16_to_f32(a.beta[bhT + tid]);
    __syncthreads();

    float S[R][CPL];
    if (valid) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t w[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                S[r][2 * j] = bf16_lo(w[j]);
                S[r][2 * j + 1] = bf16_hi(w[j]);
            }
        }
    }

    auto commit = [&]() {
        uint16_t *dst = a.pool_out + srow0 * a.Dv + col0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint4 w;
            w.x = pack_bf16x2(S[r][0], S[r][1]);
            w.y = pack_bf16x2(S[r][2], S[r][3]);
            w.z = pack_bf16x2(S[r][4], S[r][5]);
            w.w = pack_bf16x2(S[r][6], S[r][7]);
            *reinterpret_cast<uint4 *>(dst + (size_t)(rg + r * RPP) * a.Dv) = w;
        }
    };
    if (valid && n == 0) commit();

    float *ex = lds + T * Sh::TOK;
    for (int t = 0; t < L; ++t) {
        const float *tok = lds + t * Sh::TOK;
        float pk[CPL], pq[CPL], kr[R];
        float kq = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) pk[c] = pq[c] = 0.f;
        // Step 1 (decay) fused with the partial sums of steps 2 and 4.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = rg + r * RPP;
            const float d = tok[i], kk = tok[DK + i], qq = tok[2 * DK + i];
            kr[r] = kk;
            kq = fmaf(kk, qq, kq);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const float s = S[r][c] * d;
                S[r][c] = s;
                pk[c] = fmaf(s, kk, pk[c]);
                pq[c] = fmaf(s, qq, pq[c]);
            }
        }
        // Lanes of one wave holding the same columns are LPR apart.
#pragma unroll
        for (int m = LPR; m < 64; m <<= 1) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                pk[c] += __shfl_xor(pk[c], m);
                pq[c] += __shfl_xor(pq[c], m);
            }
            kq += __shfl_xor(kq, m);
        }
        float *exb = ex + (t & 1) * Sh::EX;
        if (lane < LPR) {
            float *dst = exb + wave * Sh::EXW;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                dst[cg * CPL + c] = pk[c];
                dst[TV + cg * CPL + c] = pq[c];
            }
            if (lane == 0) dst[2 * TV] = kq;
        }
        __syncthreads();
        float P[CPL], Q[CPL], KQ = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) P[c] = Q[c] = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float *src = exb + w * Sh::EXW;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                P[c] += src[cg * CPL + c];
                Q[c] += src[TV + cg * CPL + c];
            }
            KQ += src[2 * TV];
        }
        // Step 3 (delta update) and step 4 (output with the updated state).
        const float bt = tok[3 * DK + TV];
        float u[CPL], o[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            u[c] = bt * (tok[3 * DK + cg * CPL + c] - P[c]);
            o[c] = fmaf(KQ, u[c], Q[c]);
        }
        if (rg == 0) {
            uint4 w;
            w.x = pack_bf16x2(o[0], o[1]);
            w.y = pack_bf16x2(o[2], o[3]);
            w.z = pack_bf16x2(o[4], o[5]);
            w.w = pack_bf16x2(o[6], o[7]);
            *reinterpret_cast<uint4 *>(out_row + (size_t)t * a.Dv) = w;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < CPL; ++c) S[r][c] = fmaf(kr[r], u[c], S[r][c]);
        if (t + 1 == n) commit();
    }
    // Padded tokens (and skipped entries): +0.0 output rows.
    if (rg == 0)
        for (int t = L; t < T; ++t)
            *reinterpret_cast<uint4 *>(out_row + (size_t)t * a.Dv) = make_uint4(0, 0, 0, 0);
}

template <int DK, int TV>
static hipError_t launch_decode(const DecodeArgs &a, unsigned grid, hipStream_t stream) {
    constexpr int NT = 256;
    const size_t lds = TileShape<DK, TV, NT>::lds_bytes(a.T);
    hipLaunchKernelGGL((decode_kernel<DK, TV, NT>), dim3(grid), dim3(NT), lds, stream, a);
    return hipGetLastError();
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
    if (B <= 0 || H_q <= 0 || H_v <= 0 || T <= 0 || D_k <= 0 || D_v <= 0 || N_slots <= 0)
        return RGDR_ERR_SHAPE;
    if (T > kMaxT || H_v % H_q != 0) return RGDR_ERR_SHAPE;
    if ((D_k != 64 && D_k != 128) || D_v % 64 != 0) return RGDR_ERR_UNSUPPORTED;
    if (!aligned(value, 16) || !aligned(state_pool, 16) || !aligned(out, 16) ||
        !aligned(state_out, 16) || !aligned(query, 2) || !aligned(key, 2) ||
        !aligned(beta, 2) || !aligned(g, 4) || !aligned(gk, 4) ||
        !aligned(actual_seq_lengths, 4) || !aligned(ssm_state_indices, 4) ||
        !aligned(num_accepted_tokens, 4))
        return RGDR_ERR_ALIGN;

    const int tile_v = (D_v % 128 == 0) ? 128 : 64;
    const long long grid = (long long)B * H_v * (D_v / tile_v);
    if (grid > 0x7FFFFFFFLL) return RGDR_ERR_SHAPE;

    DecodeArgs a;
    a.q = static_cast<const uint16_t *>(query);
    a.k = static_cast<const uint16_t *>(key);
    a.v = static_cast<const uint16_t *>(value);
    a.beta = static_cast<const uint16_t *>(beta);
    a.pool = static_cast<const uint16_t *>(state_pool);
    a.lens = actual_seq_lengths;
    a.idx = ssm_state_indices;
    a.nacc = num_accepted_tokens;
    a.g = g;
    a.gk = gk;
    a.out = static_cast<uint16_t *>(out);
    a.pool_out = static_cast<uint16_t *>(state_out);
    a.scale = scale;
    a.Hq = H_q;
    a.Hv = H_v;
    a.T = T;
    a.Dv = D_v;
    a.N_slots = N_slots;
    a.ntiles = D_v / tile_v;
    a.group = H_v / H_q;

    hipError_t err;
    if (D_k == 128)
        err = tile_v == 128 ? launch_decode<128, 128>(a, (unsigned)grid, stream)
                            : launch_decode<128, 64>(a, (unsigned)grid, stream);
    else
        err = tile_v == 128 ? launch_decode<64, 128>(a, (unsigned)grid, stream)
                            : launch_decode<64, 64>(a, (unsigned)grid, stream);
    return err == hipSuccess ? RGDR_OK : RGDR_ERR_HIP;
}
