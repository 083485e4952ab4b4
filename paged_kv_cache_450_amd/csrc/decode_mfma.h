// Matrix-core decode math and kernel for grouped query heads on 16-bit caches.
#pragma once

#include "decode_core.h"

namespace {

using namespace pkv::dev;

// ---------------------------------------------------------------------------
// Matrix-core decode for 16-bit caches with grouped query heads.
//
// With G query heads per kv head a tile costs G times the multiply-adds of one
// head (8 flop per KV byte at G = 8), which the vector ALU cannot sustain at
// HBM rate. Here both products run on MFMA, with the G heads padded to 16:
//   S^T = K Q^T    (v_mfma 16x16x32: rows = the 16 tokens of a tile,
//                   columns = heads, contraction over 32 dims per step)
//   O^T += V^T P^T (v_mfma 16x16x16: rows = 16 dims, columns = heads,
//                   contraction over the 16 tokens of the tile)
// Lane l works for head l % 16. After the QK product it holds that head's
// scores for tokens 4*(l/16) .. +3, which is exactly the B operand P^T of the
// PV product, so the probabilities never move between lanes; the running max
// is shared by the four lanes of a head with two xor-shuffles, and the O^T
// accumulator of a lane belongs to its own head, so rescaling is lane-local.
// The A operand of the QK product wants lane l to hold token l % 16, dims
// 32c + 8 (l / 16): the streaming kernels load K in its natural layout (1 KiB
// per load, whole 128-byte lines) and move it there through an LDS K stage
// (k_operand); the prefix kernel loads it in the operand layout directly.
// V^T, the A operand of the PV product, needs each lane to hold 4 tokens of
// one dim: V goes through a per-wave LDS tile in its natural layout, and
// ds_read_tr16_b64 returns the transposed 4 x 16-bit groups (one read per 16
// dims). Row pitches 2D + 48 (D = 128) and 2D + 16 (D = 64) bytes keep both
// the row writes and the transposed reads free of bank conflicts.
// P enters the PV product in the cache dtype (bf16: as the sum of two bf16
// terms, see mfma_consume); both products accumulate in fp32.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

template <int KV>
__device__ __forceinline__ f32x4_t mfma_qk(const uint4& a, const uint4& b, f32x4_t c) {
    if constexpr (KV == PKV_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <int KV>
__device__ __forceinline__ f32x4_t mfma_pv(s16x4_t a, s16x4_t b, f32x4_t c) {
    if constexpr (KV == PKV_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

template <int D>
struct MfmaGeo {
    static constexpr int kTileBytes = 16 * D * 2;
    static constexpr int kNk = D / 32;                 // QK steps = K loads per tile
    static constexpr int kNv = D / 32;                 // 1 KiB V loads per tile
    static constexpr int kNd = D / 16;                 // PV steps per tile
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kPitch = 2 * D + (D == 128 ? 48 : 16);
    static constexpr int kStage = 16 * kPitch;         // LDS bytes of one staged V tile
};

template <int D>
struct MfmaTile {
    uint4 k[MfmaGeo<D>::kNk];
    uint4 v[MfmaGeo<D>::kNv];
};

// The Q^T operand of a wave lives in its LDS (leaving the registers to a
// deeper tile ring), chunk-major so that each per-tile read of one 32-dim
// chunk is a contiguous, conflict-free 1 KiB.
template <int D>
struct QLds {
    const uint8_t* base;  // kNk x 1 KiB
    __device__ __forceinline__ uint4 get(int c, int lane) const {
        return *reinterpret_cast<const uint4*>(base + c * 1024 + lane * 16);
    }
};

// K loaded in its natural layout (lane l of load c: bytes 1024c + 16l of the
// tile, as V is) into the QK product's A operand (token l % 16, dims
// 32c + 8 (l / 16)) through the wave's LDS K stage: rows at pitch kPitch,
// which keeps both the row writes and the column reads free of bank
// conflicts. A load of natural K touches whole 128-byte lines (8 per load)
// where the operand layout's own loads touch 64 bytes of 16 lines each.
template <int D>
__device__ __forceinline__ void k_operand(const MfmaTile<D>& t, uint8_t* kst,
                                          uint4 (&a)[MfmaGeo<D>::kNk], int lane) {
    using Gm = MfmaGeo<D>;
#pragma unroll
    for (int c = 0; c < Gm::kNk; ++c) {
        const int byte = 1024 * c + 16 * lane;
        *reinterpret_cast<uint4*>(kst + (byte / Gm::kRowBytes) * Gm::kPitch +
                                  byte % Gm::kRowBytes) = t.k[c];
    }
#pragma unroll
    for (int c = 0; c < Gm::kNk; ++c)
        a[c] = *reinterpret_cast<const uint4*>(kst + (lane & 15) * Gm::kPitch + 64 * c +
                                               16 * (lane >> 4));
}

// The first half of a tile's math, everything that reads the tile's
// registers: the scores S^T = K Q^T of head hl for tokens 4*kg + r (returned),
// and V staged in LDS (natural layout, padded rows; tokens outside
// [nlo, nvalid) become zeros so that stale or NaN bytes never meet a zero
// probability). Once it returns, the tile's registers may be refilled.
// kPartial: the masked form. kst: NULL when K was loaded in the operand
// layout, else the wave's K stage (K loaded in its natural layout).
template <int KV, int D, bool kPartial, class QSrc>
__device__ __forceinline__ f32x4_t mfma_front(const MfmaTile<D>& t, int nvalid, int nlo,
                                              const QSrc& qsrc, uint8_t* stage, int lane,
                                              uint8_t* kst = nullptr) {
    using Gm = MfmaGeo<D>;
    f32x4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (kst != nullptr) {
        uint4 a[Gm::kNk];
        k_operand<D>(t, kst, a, lane);
#pragma unroll
        for (int c = 0; c < Gm::kNk; ++c) sacc = mfma_qk<KV>(a[c], qsrc.get(c, lane), sacc);
    } else {
#pragma unroll
        for (int c = 0; c < Gm::kNk; ++c) sacc = mfma_qk<KV>(t.k[c], qsrc.get(c, lane), sacc);
    }
    constexpr int kLanesPerRow = Gm::kRowBytes / 16;
#pragma unroll
    for (int i = 0; i < Gm::kNv; ++i) {
        const int tok = i * (64 / kLanesPerRow) + lane / kLanesPerRow;
        uint4 v = t.v[i];
        if constexpr (kPartial) {
            if (tok >= nvalid || tok < nlo) v = make_uint4(0u, 0u, 0u, 0u);
        }
        *reinterpret_cast<uint4*>(stage + tok * Gm::kPitch + (lane % kLanesPerRow) * 16) = v;
    }
    return sacc;
}

// The second half: online softmax of the scores and O^T += V^T P^T from the
// staged V. Attended tokens: [nlo, nvalid).
template <int KV, int D, bool kPartial>
__device__ __forceinline__ void mfma_back(f32x4_t sacc, int nvalid, int nlo,
                                          f32x4_t (&o)[MfmaGeo<D>::kNd], float& m, float& lsum,
                                          float sscale, const uint8_t* stage, int lane) {
    using Gm = MfmaGeo<D>;
    const int kg = lane >> 4;   // this lane's tokens: 4*kg .. 4*kg + 3
    const int hl = lane & 15;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        sc[r] = sacc[r] * sscale;
        if constexpr (kPartial)
            sc[r] = (4 * kg + r < nvalid && 4 * kg + r >= nlo) ? sc[r] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // m is the reference of the exponentials. It is raised, and the sums
    // rescaled, only when a score passes it by more than kSlack (log2 units),
    // so probabilities stay below 2^kSlack and rescaling is rare: the O^T
    // accumulators live in AGPRs, where a rescale costs three instructions
    // per element.
    constexpr float kSlack = 8.0f;
    if (__ballot(mx > m + kSlack)) {
        const float mnew = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mnew);  // m = -inf: 0 (o and lsum are still 0)
        lsum *= alpha;
#pragma unroll
        for (int j = 0; j < Gm::kNd; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[j][r] *= alpha;
        m = mnew;
    }
    const float ms = (m == -INFINITY) ? 0.0f : m;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sc[r] - ms);
    lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const s16x4_t pb = __builtin_bit_cast(
        s16x4_t, make_uint2(pack2<KV>(pr[0], pr[1]), pack2<KV>(pr[2], pr[3])));
    // bf16 keeps 8 bits of a probability, which can leave a product with one
    // dominant token 2^-9 of |v| off; the rounding residual goes through a
    // second product, so P enters exact to about 2^-17. (f16 keeps 11 bits.)
    s16x4_t pb_lo = {0, 0, 0, 0};
    if constexpr (KV == PKV_BF16) {
        float rl[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            rl[r] = pr[r] - __builtin_bit_cast(float, static_cast<uint32_t>(
                                                          static_cast<uint16_t>(pb[r])) << 16);
        pb_lo = __builtin_bit_cast(s16x4_t,
                                   make_uint2(pack2<KV>(rl[0], rl[1]), pack2<KV>(rl[2], rl[3])));
    }
    // Transposed reads: lane (within its group of 16) j' supplies row
    // 4*kg + j'/4, dims 16*jd + 4*(j'%4); it receives dims 16*jd + j' of
    // tokens 4*kg .. 4*kg + 3.
    const uint8_t* rd = stage + (4 * kg + (hl >> 2)) * Gm::kPitch + 8 * (hl & 3);
#pragma unroll
    for (int jd = 0; jd < Gm::kNd; ++jd) {
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        const v4i16 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(rd + 32 * jd));
        o[jd] = mfma_pv<KV>(__builtin_bit_cast(s16x4_t, va), pb, o[jd]);
        if constexpr (KV == PKV_BF16) o[jd] = mfma_pv<KV>(__builtin_bit_cast(s16x4_t, va), pb_lo, o[jd]);
    }
}

// One tile's whole math. Attended tokens of the tile: [nlo, nvalid)
// (kPartial: the masked form).
template <int KV, int D, bool kPartial, class QSrc>
__device__ __forceinline__ void mfma_consume(const MfmaTile<D>& t, int nvalid, int nlo,
                                             const QSrc& qsrc,
                                             f32x4_t (&o)[MfmaGeo<D>::kNd], float& m, float& lsum,
                                             float sscale, uint8_t* stage, int lane,
                                             uint8_t* kst = nullptr) {
    const f32x4_t sacc = mfma_front<KV, D, kPartial>(t, nvalid, nlo, qsrc, stage, lane, kst);
    mfma_back<KV, D, kPartial>(sacc, nvalid, nlo, o, m, lsum, sscale, stage, lane);
}

template <int KV, int D, int G, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(const DecodeParams p) {
    using Gm = MfmaGeo<D>;
    constexpr int NK = Gm::kNk, NV = Gm::kNv, ND = Gm::kNd, TB = Gm::kTileBytes;
    static_assert(G >= 1 && G <= 16, "heads padded to 16");

    const int g = blockIdx.x;
    const int part = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int w = (NW == 1) ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane & 15;
    const int kg = lane >> 4;

    WaveWork ww;
    if (!locate_work<G, D, NW>(p, g, part, w, ww)) return;
    const int s = ww.s, L = ww.L, n = ww.n;
    BlockIds<NW> ids;
    ids.init(p.block_tables + static_cast<size_t>(s) * p.max_blocks + ww.b0, n, lane);

    // Q^T operand in the wave's LDS: head hl (zeros for the padding heads),
    // dims 32c + 8*kg .. +8. Padding lanes read head G-1 (always inside q) and
    // discard it.
    __shared__ __attribute__((aligned(16))) uint8_t q_all[NW][NK * 1024];
    const QLds<D> qr{q_all[w]};
    {
        const int hq = g * G + min(hl, G - 1);
        const uint16_t* qrow =
            static_cast<const uint16_t*>(p.q) + (static_cast<size_t>(s) * p.num_q_heads + hq) * D;
        uint4 qv[NK];
#pragma unroll
        for (int c = 0; c < NK; ++c) qv[c] = *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * kg);
#pragma unroll
        for (int c = 0; c < NK; ++c)
            *reinterpret_cast<uint4*>(q_all[w] + c * 1024 + lane * 16) =
                hl < G ? qv[c] : make_uint4(0u, 0u, 0u, 0u);
    }
    const float sscale = p.scale_log2;
    f32x4_t o[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j) o[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, lsum = 0.0f;

    __shared__ __attribute__((aligned(16))) uint8_t stage_all[NW][Gm::kStage];
    __shared__ __attribute__((aligned(16))) uint8_t kst_all[NW][Gm::kStage];
    uint8_t* stage = stage_all[w];
    uint8_t* kst = kst_all[w];

    const uint8_t* kpl = p.k_plane + static_cast<size_t>(g) * TB;
    const uint8_t* vpl = p.v_plane + static_cast<size_t>(g) * TB;
    const size_t bstride = static_cast<size_t>(p.num_kv_heads) * TB;
    const int voff = lane * 16;  // + 1024*i: K and V in natural rows (K to its operand via kst)

    MfmaTile<D> t[NBUF];
    int nv[NBUF], nl[NBUF];
    auto issue = [&](MfmaTile<D>& tt, int& nvalid, int& nlo, int kn) {
        const TileRef r = tile_ref(p, kpl, vpl, bstride, TB, ids.next(kn), (ww.b0 + kn * NW) * 16,
                                   L, ww.lo);
        nvalid = r.nvalid;
        nlo = r.nlo;
#pragma unroll
        for (int c = 0; c < NK; ++c) tt.k[c] = rsrc_load16(r.k, voff + 1024 * c);
#pragma unroll
        for (int i = 0; i < NV; ++i) tt.v[i] = rsrc_load16(r.v, voff + 1024 * i);
    };

#pragma unroll
    for (int x = 0; x < NBUF; ++x) issue(t[x], nv[x], nl[x], x);
    for (int k0 = 0; k0 < n; k0 += NBUF) {
#pragma unroll
        for (int x = 0; x < NBUF; ++x) {
            if (nv[x] == 16 && nl[x] == 0)
                mfma_consume<KV, D, false>(t[x], 16, 0, qr, o, m, lsum, sscale, stage, lane, kst);
            else
                mfma_consume<KV, D, true>(t[x], nv[x], nl[x], qr, o, m, lsum, sscale, stage, lane,
                                          kst);
            issue(t[x], nv[x], nl[x], k0 + x + NBUF);
        }
    }

    // The four lanes of a head share m; their partial sums add up to l.
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);

    if constexpr (NW == 1) {
        if (hl < G) {
            const int qh = g * G + hl;
            const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
            if (p.blocks_per_part > 0) {
                const size_t slot = (static_cast<size_t>(s) * p.num_q_heads + qh) * p.num_parts + part;
                float* dst = p.ws_o + slot * D + 4 * kg;
#pragma unroll
                for (int j = 0; j < ND; ++j)
                    *reinterpret_cast<float4*>(dst + 16 * j) =
                        make_float4(o[j][0] * inv, o[j][1] * inv, o[j][2] * inv, o[j][3] * inv);
                if (kg == 0) store_ml(p, s, qh, part, m, lsum);
            } else {
                uint16_t* dst = static_cast<uint16_t*>(p.out) +
                                (static_cast<size_t>(s) * p.num_q_heads + qh) * D + 4 * kg;
#pragma unroll
                for (int j = 0; j < ND; ++j)
                    *reinterpret_cast<uint2*>(dst + 16 * j) =
                        make_uint2(pack2<KV>(o[j][0] * inv, o[j][1] * inv),
                                   pack2<KV>(o[j][2] * inv, o[j][3] * inv));
            }
        }
    } else {
        __shared__ float lds_o[NW][G][D];
        __shared__ float lds_m[NW][G];
        __shared__ float lds_l[NW][G];
        if (hl < G) {
#pragma unroll
            for (int j = 0; j < ND; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) lds_o[w][hl][16 * j + 4 * kg + r] = o[j][r];
            if (kg == 0) {
                lds_m[w][hl] = m;
                lds_l[w][hl] = lsum;
            }
        }
        __syncthreads();
        combine_waves<KV, D, G, NW>(p, s, g, part, lds_o, lds_m, lds_l, 1.0f);
    }
}

}  // namespace
