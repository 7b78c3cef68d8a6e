// rgdr_host.cpp -- host-only parts of the C ABI: index validation and status names.
//
// The decode step (MindSpore Lite page "lite_boost.ops.recurrent_gated_delta_rule",
// parameter list) takes per-entry valid lengths, accepted-token counts and slot indices
// into a global state pool. The kernel never leaves its buffers whatever these hold; the
// checks below tell a caller when they break the call's preconditions.
#include <hip/hip_runtime.h>

#include <vector>

#include "rgdr.h"

extern "C" rgdr_status rgdr_validate_host(const int32_t *actual_seq_lengths,
                                          const int32_t *ssm_state_indices,
                                          const int32_t *num_accepted_tokens, int32_t B,
                                          int32_t T, int32_t N_slots) {
    if (!actual_seq_lengths || !ssm_state_indices || !num_accepted_tokens)
        return RGDR_ERR_NULL;
    if (B <= 0 || T <= 0 || N_slots <= 0) return RGDR_ERR_SHAPE;
    std::vector<unsigned char> seen((size_t)N_slots, 0);
    rgdr_status st = RGDR_OK;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t L = actual_seq_lengths[b];
        const int32_t n = num_accepted_tokens[b];
        const int32_t s = ssm_state_indices[b];
        if (L < 0 || L > T || n < 0 || n > L || s < 0 || s >= N_slots) return RGDR_ERR_RANGE;
        if (seen[(size_t)s]) st = RGDR_ERR_DUPLICATE;
        seen[(size_t)s] = 1;
    }
    return st;
}

extern "C" rgdr_status rgdr_validate(const int32_t *actual_seq_lengths,
                                     const int32_t *ssm_state_indices,
                                     const int32_t *num_accepted_tokens, int32_t B, int32_t T,
                                     int32_t N_slots, hipStream_t stream) {
    if (!actual_seq_lengths || !ssm_state_indices || !num_accepted_tokens)
        return RGDR_ERR_NULL;
    if (B <= 0 || T <= 0 || N_slots <= 0) return RGDR_ERR_SHAPE;
    std::vector<int32_t> h((size_t)3 * B);
    const size_t bytes = sizeof(int32_t) * (size_t)B;
    if (hipMemcpyAsync(h.data(), actual_seq_lengths, bytes, hipMemcpyDeviceToHost, stream) !=
            hipSuccess ||
        hipMemcpyAsync(h.data() + B, ssm_state_indices, bytes, hipMemcpyDeviceToHost, stream) !=
            hipSuccess ||
        hipMemcpyAsync(h.data() + 2 * (size_t)B, num_accepted_tokens, bytes,
                       hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return RGDR_ERR_HIP;
    return rgdr_validate_host(h.data(), h.data() + B, h.data() + 2 * (size_t)B, B, T, N_slots);
}

extern "C" const char *rgdr_status_string(rgdr_status s) {
    switch (s) {
    case RGDR_OK: return "RGDR_OK";
    case RGDR_ERR_NULL: return "RGDR_ERR_NULL: a required pointer is NULL";
    case RGDR_ERR_SHAPE: return "RGDR_ERR_SHAPE: invalid size (<= 0, T > 8, H_v % H_q != 0, "
                                "grid too large, or beta requested without b)";
    case RGDR_ERR_UNSUPPORTED: return "RGDR_ERR_UNSUPPORTED: D_k must be 64 or 128 and D_v a "
                                      "multiple of 64 up to 4096; unknown option bit";
    case RGDR_ERR_RANGE: return "RGDR_ERR_RANGE: a length, accepted count or slot index is out "
                                "of range";
    case RGDR_ERR_DUPLICATE: return "RGDR_ERR_DUPLICATE: two batch entries name the same slot";
    case RGDR_ERR_DTYPE: return "RGDR_ERR_DTYPE: dtype not allowed for this argument";
    case RGDR_ERR_HIP: return "RGDR_ERR_HIP: a HIP runtime call failed";
    case RGDR_ERR_ALIGN: return "RGDR_ERR_ALIGN: a pointer is not aligned as required";
    case RGDR_ERR_SCRATCH: return "RGDR_ERR_SCRATCH: the call needs more scratch memory than "
                                  "rgdr_prefill_noalloc's fixed 128 MiB array";
    }
    return "unknown rgdr_status";
}
