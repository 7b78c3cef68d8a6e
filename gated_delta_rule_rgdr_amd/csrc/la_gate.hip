// la_gate.hip -- the linear-attention gate front end on gfx950.
//
// Method: kernel README "com.microsoft.LinearAttentionGate" (Description; Inputs, Outputs
// and Type constraints tables): decay = decay_scale[h] * softplus(a + dt_bias[h]) and,
// when requested, beta = sigmoid(b); the head axis is last, leading axes are folded;
// arithmetic is fp32 and values are narrowed only on store.
//
// An elementwise, bandwidth-trivial kernel: each thread handles elements strided by the
// grid, reads a (and b) once, writes decay (and beta) once. softplus uses the overflow-safe
// form x + log1p(e^-x) (x > 0) / log1p(e^x), which is the same function.
#include "rgdr_common.h"

namespace rgdr {

struct GateArgs {
    const void *a, *b;
    const float *dt_bias, *decay_scale;
    void *decay, *beta;
    long long n;
    int H;
    int decay_dtype, beta_dtype;
};

template <typename TIn>
__device__ __forceinline__ float load_in(const void *p, long long e) {
    return static_cast<float>(static_cast<const TIn *>(p)[e]);
}

__device__ __forceinline__ void store_out(void *p, int dtype, long long e, float x) {
    if (dtype == RGDR_F32)
        static_cast<float *>(p)[e] = x;
    else if (dtype == RGDR_F16)
        static_cast<_Float16 *>(p)[e] = static_cast<_Float16>(x);
    else
        static_cast<uint16_t *>(p)[e] = f32_to_bf16(x);
}

template <typename TIn>
__global__ __launch_bounds__(256) void la_gate_kernel(const GateArgs g) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < g.n; e += stride) {
        const int h = (int)(e % g.H);
        const float x = load_in<TIn>(g.a, e) + g.dt_bias[h];
        store_out(g.decay, g.decay_dtype, e, g.decay_scale[h] * softplus_f32(x));
        if (g.beta) store_out(g.beta, g.beta_dtype, e, sigmoid_f32(load_in<TIn>(g.b, e)));
    }
}

static size_t dtype_size(int d) { return d == RGDR_F32 ? 4 : 2; }

}  // namespace rgdr

extern "C" rgdr_status la_gate(const void *a, const float *dt_bias, const float *decay_scale,
                               const void *b, rgdr_dtype ab_dtype, int64_t n_rows, int32_t H,
                               void *decay_out, rgdr_dtype decay_dtype, void *beta_out,
                               rgdr_dtype beta_dtype, hipStream_t stream) {
    using namespace rgdr;
    if (n_rows < 0 || H <= 0) return RGDR_ERR_SHAPE;
    if (ab_dtype != RGDR_F32 && ab_dtype != RGDR_F16) return RGDR_ERR_DTYPE;
    if (decay_dtype != RGDR_F32 && decay_dtype != RGDR_F16) return RGDR_ERR_DTYPE;
    if (beta_out && beta_dtype != RGDR_F32 && beta_dtype != RGDR_F16 && beta_dtype != RGDR_BF16)
        return RGDR_ERR_DTYPE;
    if (beta_out && !b) return RGDR_ERR_SHAPE;
    long long n = 0;
    if (__builtin_mul_overflow((long long)n_rows, (long long)H, &n)) return RGDR_ERR_SHAPE;
    if (n == 0) return RGDR_OK;  // empty input: nothing to do, no pointer is read
    if (!a || !dt_bias || !decay_scale || !decay_out) return RGDR_ERR_NULL;
    const size_t in_sz = dtype_size(ab_dtype);
    if (!aligned(a, in_sz) || (b && !aligned(b, in_sz)) || !aligned(dt_bias, 4) ||
        !aligned(decay_scale, 4) || !aligned(decay_out, dtype_size(decay_dtype)) ||
        (beta_out && !aligned(beta_out, dtype_size(beta_dtype))))
        return RGDR_ERR_ALIGN;

    GateArgs g;
    g.a = a;
    g.b = beta_out ? b : nullptr;
    g.dt_bias = dt_bias;
    g.decay_scale = decay_scale;
    g.decay = decay_out;
    g.beta = beta_out;
    g.n = n;
    g.H = H;
    g.decay_dtype = decay_dtype;
    g.beta_dtype = beta_dtype;
    constexpr int NT = 256;
    // Enough workgroups to cover every element once, capped at a few per CU (grid-stride
    // loop beyond that).
    const long long want = (n + NT - 1) / NT;
    const unsigned grid = (unsigned)(want < 2048 ? want : 2048);
    if (ab_dtype == RGDR_F32)
        hipLaunchKernelGGL(la_gate_kernel<float>, dim3(grid), dim3(NT), 0, stream, g);
    else
        hipLaunchKernelGGL(la_gate_kernel<_Float16>, dim3(grid), dim3(NT), 0, stream, g);
    return hipGetLastError() == hipSuccess ? RGDR_OK : RGDR_ERR_HIP;
}
