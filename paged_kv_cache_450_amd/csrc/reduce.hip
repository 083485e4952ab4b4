// paged_attn_reduce: merge the split-K partitions of a partitioned decode.
//
// Long contexts are cut into partitions of partition_size tokens so that the
// work per workgroup stays bounded whatever the context length (the pages'
// long-context pressure is [P2] "vLLM 也不是银弹：真实部署中的坑", third pitfall).
// Partition p leaves m_p (max score), l_p (sum of exp(s - m_p)) and the
// normalised o_p; the exact merge is
//     M = max_p m_p,  w_p = l_p exp(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
//
// One wave64 per (query head, sequence). Lanes read up to 64 partitions'
// (m, l) at once, reduce M and sum w across the wave, then walk the
// partitions with each lane owning D/64 output dims (a 256- or 512-byte
// coalesced read of o_p per partition). Traffic is (D + 2) * 4 bytes per
// (sequence, head, partition), small next to the KV bytes the decode reads.

#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "device.h"

namespace {

using namespace pkv::dev;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <int OUT, int D>
__global__ __launch_bounds__(64) void reduce_kernel(const float* __restrict__ ml,
                                                    const float* __restrict__ o,
                                                    uint16_t* __restrict__ out,
                                                    const int32_t* __restrict__ lens,
                                                    int32_t num_q_heads, int32_t P, int32_t PS,
                                                    int32_t max_ctx) {
    constexpr int DPL = D / 64;
    const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
    int L = min(lens[s], max_ctx);
    const int np = L > 0 ? (L + PS - 1) / PS : 0;
    const size_t base = (static_cast<size_t>(s) * num_q_heads + h) * P;

    // The first 64 partitions' (m, l) stay in registers for the weights (one
    // load of them for contexts of up to 64 partitions).
    float m0 = -INFINITY, l0 = 0.0f;
    if (lane < np) {
        m0 = ml[(base + lane) * 2];
        l0 = ml[(base + lane) * 2 + 1];
    }
    float mloc = m0;
    for (int p0 = 64; p0 < np; p0 += 64)
        if (p0 + lane < np) mloc = fmaxf(mloc, ml[(base + p0 + lane) * 2]);
    const float M = wave_max(mloc);

    float acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
    float wsum = 0.0f;
    if (M != -INFINITY) {
        for (int p0 = 0; p0 < np; p0 += 64) {
            float wl = 0.0f;
            if (p0 + lane < np) {
                const float mp = p0 == 0 ? m0 : ml[(base + p0 + lane) * 2];
                const float lp = p0 == 0 ? l0 : ml[(base + p0 + lane) * 2 + 1];
                wl = lp * expf(mp - M);
            }
            wsum += wl;
            const int cnt = min(64, np - p0);
            // kRound partitions per round: their o loads are all issued before
            // the first is used (one memory latency per round, not per partition).
            constexpr int kRound = 32;
            for (int k0 = 0; k0 < cnt; k0 += kRound) {
                float ov[kRound][DPL];
#pragma unroll
                for (int u = 0; u < kRound; ++u) {
                    const float* op = o + (base + p0 + min(k0 + u, cnt - 1)) * D + lane * DPL;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) ov[u][e] = op[e];
                }
#pragma unroll
                for (int u = 0; u < kRound; ++u) {
                    // partitions past cnt re-read the last one and get weight 0
                    const float wk = k0 + u < cnt
                                         ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                         __builtin_bit_cast(int, wl),
                                                                         k0 + u))
                                         : 0.0f;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wk, ov[u][e], acc[e]);
                }
            }
        }
    }
    const float W = wave_sum(wsum);
    const size_t ob = (static_cast<size_t>(s) * num_q_heads + h) * D + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        const float r = W > 0.0f ? acc[e] / W : 0.0f;
        out[ob + e] = (OUT == PKV_F16) ? f32_to_f16_bits(r) : f32_to_bf16_bits(r);
    }
}

template <int OUT, int D>
hipError_t launch(const float* ml, const float* o, void* out, const int32_t* lens, int32_t B,
                  int32_t Hq, int32_t P, int32_t PS, int32_t max_ctx, hipStream_t st) {
    hipLaunchKernelGGL((reduce_kernel<OUT, D>), dim3(Hq, B), dim3(64), 0, st, ml, o,
                       static_cast<uint16_t*>(out), lens, Hq, P, PS, max_ctx);
    return hipGetLastError();
}

}  // namespace

extern "C" pkv_status paged_attn_reduce(const void* workspace, void* out, int32_t out_dtype,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t head_dim,
                                        int32_t max_context_len, int32_t partition_size,
                                        hipStream_t stream) {
    using pkv::fail;
    if (!pkv::is_16bit(out_dtype))
        return fail(PKV_ERR_INVALID, "paged_attn_reduce: out dtype must be F16 or BF16");
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_ERR_INVALID, "paged_attn_reduce: head_dim %d not 64 or 128", head_dim);
    if (partition_size <= 0 || partition_size % 16 != 0)
        return fail(PKV_ERR_INVALID, "paged_attn_reduce: partition_size %d", partition_size);
    if (num_seqs < 0 || num_seqs > 65535 || num_q_heads <= 0 || max_context_len < 0)
        return fail(PKV_ERR_INVALID, "paged_attn_reduce: bad sizes");
    if (num_seqs == 0) return PKV_OK;
    if (out == nullptr || context_lens == nullptr)
        return fail(PKV_ERR_INVALID, "paged_attn_reduce: NULL out or context_lens");
    const int64_t P = (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
    if (P > 0 && workspace == nullptr)
        return fail(PKV_ERR_INVALID, "paged_attn_reduce: workspace is NULL");
    const float* ml = static_cast<const float*>(workspace);
    const float* o = ml == nullptr ? nullptr
                                   : reinterpret_cast<const float*>(
                                         static_cast<const uint8_t*>(workspace) +
                                         pkv::ws_o_offset(num_seqs, num_q_heads, P));
    hipError_t e;
    const int32_t Pi = static_cast<int32_t>(P);
    if (out_dtype == PKV_F16)
        e = head_dim == 64
                ? launch<PKV_F16, 64>(ml, o, out, context_lens, num_seqs, num_q_heads, Pi,
                                      partition_size, max_context_len, stream)
                : launch<PKV_F16, 128>(ml, o, out, context_lens, num_seqs, num_q_heads, Pi,
                                       partition_size, max_context_len, stream);
    else
        e = head_dim == 64
                ? launch<PKV_BF16, 64>(ml, o, out, context_lens, num_seqs, num_q_heads, Pi,
                                       partition_size, max_context_len, stream)
                : launch<PKV_BF16, 128>(ml, o, out, context_lens, num_seqs, num_q_heads, Pi,
                                        partition_size, max_context_len, stream);
    if (e != hipSuccess)
        return fail(PKV_ERR_HIP, "paged_attn_reduce: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}
