// Shared-prefix pass: the leading blocks a group of sequences shares, read once
// for all the group's members, on matrix cores.
#pragma once

#include "decode_core.h"
#include "decode_mfma.h"

namespace {

using namespace pkv::dev;

// ---------------------------------------------------------------------------
// Sequences that share a prompt map the same physical blocks ([P2]
// "PagedAttention：...": shared blocks, reference counts), so those blocks hold
// the same K/V for every member. A decode that reads them per member moves
// them from HBM once per member; here they are read once per group.
//
// The matrix-core product has 16 query columns. One workgroup serves 16 query
// rows of one kv head g: 16 / G members of a group times their G heads
// (G = 1: sixteen members, G = 8: two). Its NW waves deal the group's shared
// blocks round robin, stream them through a ring of tiles exactly as the
// matrix-core decode does (decode_mfma.h), and merge through LDS into one
// partial (o / l, m in log2 units, l) per member and query head, written to
// pre[s][qh]. The balanced pass then reads each member from the first block
// after the shared ones, and its merge kernel folds the prefix partial in with
// the log-sum-exp rule (exact in real arithmetic).
//
// All workgroups of one (group, kv head) read the same tiles, so they are
// placed on one XCD: workgroups are dealt to the 8 XCDs round robin by linear
// index, and the index is laid out so that all those of a (group, kv head)
// pair share their index mod 8, and the tiles are loaded with the default
// cache policy (not the streaming one of the other decode kernels). The first
// to ask for a tile brings it into that XCD's L2 and the others find it there.
template <int KV, int D, int G, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void prefix_kernel(const DecodeParams p) {
    using Gm = MfmaGeo<D>;
    constexpr int NK = Gm::kNk, NV = Gm::kNv, ND = Gm::kNd, TB = Gm::kTileBytes;
    constexpr int MPS = 16 / G;  // members per workgroup
    constexpr int SS = D + 4;
    static_assert(G >= 1 && G <= 16 && 16 % G == 0, "16 query rows per workgroup");

    // Linear index = ((pair / 8) * slots + slot) * 8 + pair % 8, pair = group * Hkv + g.
    const int bid = blockIdx.x;
    const int rest = bid >> 3;
    const int slot = rest % p.pre_slots;
    const int pair = (rest / p.pre_slots) * 8 + (bid & 7);
    if (pair >= p.num_groups * p.num_kv_heads) return;
    const int gr = pair / p.num_kv_heads, g = pair % p.num_kv_heads;
    const int m0 = p.group_offsets[gr];
    const int msz = p.group_offsets[gr + 1] - m0;
    // A plan lists each sequence at most once: members stay inside the batch.
    if (m0 < 0 || msz <= 0 || m0 + msz > p.num_seqs || slot * MPS >= msz) return;
    // Shared blocks, read through the first member's table row; a member index
    // outside the batch is skipped (its rows get zeros and no store).
    const int P = min(max(p.group_blocks[gr], 0), p.max_blocks);
    const int s0 = p.group_members[m0];
    if (static_cast<uint32_t>(s0) >= static_cast<uint32_t>(p.num_seqs)) return;

    const int lane = threadIdx.x & 63;
    const int w = (NW == 1) ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane & 15;
    const int kg = lane >> 4;

    // Q^T operand, one copy for the workgroup: row hl is head hl % G of member
    // slot*MPS + hl / G (zeros past the group's end; those lanes read the last
    // member's row and discard it). Wave c < NK writes its 32-dim chunk c.
    static_assert(NW >= NK, "one wave per Q chunk");
    __shared__ __attribute__((aligned(16))) uint8_t q_lds[NK * 1024];
    const QLds<D> qr{q_lds};
    if (w < NK) {
        const int mi = slot * MPS + hl / G;
        int s = p.group_members[m0 + min(mi, msz - 1)];
        const bool live = mi < msz && static_cast<uint32_t>(s) < static_cast<uint32_t>(p.num_seqs);
        if (!live) s = s0;
        const int hq = g * G + hl % G;
        const uint16_t* qrow =
            static_cast<const uint16_t*>(p.q) + (static_cast<size_t>(s) * p.num_q_heads + hq) * D;
        const uint4 qv = *reinterpret_cast<const uint4*>(qrow + 32 * w + 8 * kg);
        *reinterpret_cast<uint4*>(q_lds + w * 1024 + lane * 16) =
            live ? qv : make_uint4(0u, 0u, 0u, 0u);
    }

    // This wave's tiles: blocks w, w + NW, ... below P.
    const int n = P > w ? (P - w + NW - 1) / NW : 0;
    BlockIds<NW> ids;
    ids.init(p.block_tables + static_cast<size_t>(s0) * p.max_blocks + w, n, lane);

    const float sscale = p.scale_log2;
    f32x4_t o[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j) o[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, lsum = 0.0f;

    // The waves' V staging tiles during the stream; afterwards the same bytes
    // hold the waves' partials for the merge.
    constexpr int kMergeBytes = NW * 16 * (D + 2) * 4;
    constexpr int kLdsBytes = NW * Gm::kStage > kMergeBytes ? NW * Gm::kStage : kMergeBytes;
    __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kLdsBytes];
    uint8_t* stage = lds_raw + w * Gm::kStage;

    const uint8_t* kpl = p.k_plane + static_cast<size_t>(g) * TB;
    const uint8_t* vpl = p.v_plane + static_cast<size_t>(g) * TB;
    const size_t bstride = static_cast<size_t>(p.num_kv_heads) * TB;
    const int koff = hl * Gm::kRowBytes + 16 * kg;
    const int voff = lane * 16;

    MfmaTile<D> t[NBUF];
    int nv[NBUF];
    auto issue = [&](MfmaTile<D>& tt, int& nvalid, int kn) {
        // Shared blocks are full: every token of a tile is attended.
        const TileRef r =
            tile_ref(p, kpl, vpl, bstride, TB, ids.next(kn), (w + kn * NW) * 16, P * 16, 0);
        nvalid = r.nvalid;
        // Default cache policy: the other workgroups of this (group, kv head),
        // on the same XCD, read the same tiles from its L2.
#pragma unroll
        for (int c = 0; c < NK; ++c) tt.k[c] = rsrc_load16_kept(r.k, koff + 64 * c);
#pragma unroll
        for (int i = 0; i < NV; ++i) tt.v[i] = rsrc_load16_kept(r.v, voff + 1024 * i);
    };

#pragma unroll
    for (int x = 0; x < NBUF; ++x) issue(t[x], nv[x], x);
    __syncthreads();  // Q is in LDS
    for (int k0 = 0; k0 < n; k0 += NBUF) {
#pragma unroll
        for (int x = 0; x < NBUF; ++x) {
            if (nv[x] == 16)
                mfma_consume<KV, D, false>(t[x], 16, 0, qr, o, m, lsum, sscale, stage, lane);
            else if (nv[x] > 0)  // an id outside the pool: no tokens
                mfma_consume<KV, D, true>(t[x], nv[x], 0, qr, o, m, lsum, sscale, stage, lane);
            issue(t[x], nv[x], k0 + x + NBUF);
        }
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);

    // Merge the NW waves' partials of the 16 rows and store them per member.
    __syncthreads();  // every wave is done with its staging tile
    float (*lds_o)[16][D] = reinterpret_cast<float (*)[16][D]>(lds_raw);
    float (*lds_m)[16] = reinterpret_cast<float (*)[16]>(lds_raw + NW * 16 * D * 4);
    float (*lds_l)[16] = reinterpret_cast<float (*)[16]>(lds_raw + NW * 16 * (D + 1) * 4);
#pragma unroll
    for (int j = 0; j < ND; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) lds_o[w][hl][16 * j + 4 * kg + r] = o[j][r];
    if (kg == 0) {
        lds_m[w][hl] = m;
        lds_l[w][hl] = lsum;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * D; idx += NW * 64) {
        const int r = idx / D, d = idx % D;
        const int mi = slot * MPS + r / G;
        if (mi >= msz) continue;
        float mx = -INFINITY;
#pragma unroll
        for (int x = 0; x < NW; ++x) mx = fmaxf(mx, lds_m[x][r]);
        const float ms = (mx == -INFINITY) ? 0.0f : mx;
        float l = 0.0f, acc = 0.0f;
#pragma unroll
        for (int x = 0; x < NW; ++x) {
            const float a = fast_exp2(lds_m[x][r] - ms);
            l = fmaf(lds_l[x][r], a, l);
            acc = fmaf(lds_o[x][r][d], a, acc);
        }
        const int s = p.group_members[m0 + mi];
        if (static_cast<uint32_t>(s) >= static_cast<uint32_t>(p.num_seqs)) continue;
        float* dst = p.pre + (static_cast<size_t>(s) * p.num_q_heads + g * G + r % G) * SS;
        dst[d] = l > 0.0f ? acc / l : 0.0f;
        if (d == 0) {
            dst[D] = mx;
            dst[D + 1] = l;
        }
    }
}

// The shared-prefix kernel: eight waves per 16 query rows (the shared run is
// streamed by the waves in turn, so more waves mean fewer ring rounds each:
// 5% faster than four on 256 shared blocks), the matrix-core ring depths
// (three tiles at D = 128, four at D = 64).
template <int KV, int D, int G>
hipError_t launch_prefix(const DecodeParams& prm, hipStream_t st) {
    constexpr int R = (D == 128) ? 3 : 4;
    constexpr int NW = 8;
    const uint32_t pairs = static_cast<uint32_t>(prm.num_groups) * prm.num_kv_heads;
    const uint32_t wgs = (pairs + 7) / 8 * 8 * static_cast<uint32_t>(prm.pre_slots);
    hipLaunchKernelGGL((prefix_kernel<KV, D, G, NW, R>), dim3(wgs), dim3(NW * 64), 0, st, prm);
    return hipGetLastError();
}

template <int KV>
hipError_t prefix_by_shape(int D, int G, const DecodeParams& prm, hipStream_t st) {
    if (D == 64) {
        switch (G) {
            case 1: return launch_prefix<KV, 64, 1>(prm, st);
            case 2: return launch_prefix<KV, 64, 2>(prm, st);
            case 4: return launch_prefix<KV, 64, 4>(prm, st);
            default: return launch_prefix<KV, 64, 8>(prm, st);
        }
    }
    switch (G) {
        case 1: return launch_prefix<KV, 128, 1>(prm, st);
        case 2: return launch_prefix<KV, 128, 2>(prm, st);
        case 4: return launch_prefix<KV, 128, 4>(prm, st);
        default: return launch_prefix<KV, 128, 8>(prm, st);
    }
}

}  // namespace
