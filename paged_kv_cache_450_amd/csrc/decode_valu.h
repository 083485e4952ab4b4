// Vector-ALU decode math and kernel (one query head per kv head on 16-bit
// caches, and every FP8 cache): coalesced 16-byte tile loads, packed dot2 or
// hardware FP8 conversion, DPP row reductions, online softmax per lane.
#pragma once

#include "decode_core.h"

namespace {

using namespace pkv::dev;

template <int KV, int D>
struct Geo {
    static constexpr int kEsz = (KV == PKV_FP8_E4M3) ? 1 : 2;
    static constexpr int kEpl = 16 / kEsz;     // elements per lane per load
    static constexpr int kLpt = D / kEpl;      // lanes per token row
    static constexpr int kTpi = 64 / kLpt;     // tokens per wave load
    static constexpr int kNld = 16 / kTpi;     // wave loads per tile
    static constexpr int kTileBytes = 16 * D * kEsz;
    static_assert(kLpt >= 2 && kLpt <= 16 && kNld >= 1, "geometry");
};

// Query slice of one head for one lane: raw 16-bit pairs for 16-bit caches,
// fp32 values for FP8 caches.
template <int KV, int D>
struct QSlice {
    static constexpr int kEpl = Geo<KV, D>::kEpl;
    static constexpr int kWords = (KV == PKV_FP8_E4M3) ? kEpl : kEpl / 2;
    float f[(KV == PKV_FP8_E4M3) ? kEpl : 1];
    uint32_t w[(KV == PKV_FP8_E4M3) ? 1 : kEpl / 2];
};

template <int QD>
__device__ __forceinline__ void to_f32x2(uint32_t w, float& a, float& b) {
    if constexpr (QD == PKV_F16) {
        a = f16_lo(w);
        b = f16_hi(w);
    } else {
        a = bf16_lo(w);
        b = bf16_hi(w);
    }
}

template <int KV, int QD, int D>
__device__ __forceinline__ void load_q(QSlice<KV, D>& qs, const uint16_t* qrow, int col) {
    constexpr int kEpl = Geo<KV, D>::kEpl;
    const uint4* p = reinterpret_cast<const uint4*>(qrow + col * kEpl);
    if constexpr (KV != PKV_FP8_E4M3) {
        const uint4 x = p[0];
        qs.w[0] = x.x; qs.w[1] = x.y; qs.w[2] = x.z; qs.w[3] = x.w;
    } else {
#pragma unroll
        for (int c = 0; c < kEpl / 8; ++c) {
            const uint4 x = p[c];
            const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) to_f32x2<QD>(ws[i], qs.f[c * 8 + 2 * i], qs.f[c * 8 + 2 * i + 1]);
        }
    }
}

// Partial dot product of one lane's 16-byte K slice with its query slice.
template <int KV, int D>
__device__ __forceinline__ float qk_partial(const uint4& k, const QSlice<KV, D>& qs) {
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
    float acc = 0.0f;
    if constexpr (KV == PKV_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, kw[i]),
                                         __builtin_bit_cast(half2_t, qs.w[i]), acc, false);
    } else if constexpr (KV == PKV_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, kw[i]),
                                                  __builtin_bit_cast(bf162_t, qs.w[i]), acc,
                                                  false);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float2_t lo = e4m3x2_lo(kw[i]);
            const float2_t hi = e4m3x2_hi(kw[i]);
            acc = fmaf(lo.x, qs.f[4 * i + 0], acc);
            acc = fmaf(lo.y, qs.f[4 * i + 1], acc);
            acc = fmaf(hi.x, qs.f[4 * i + 2], acc);
            acc = fmaf(hi.y, qs.f[4 * i + 3], acc);
        }
    }
    return acc;
}

// One lane's 16-byte V slice as fp32.
template <int KV, int D>
__device__ __forceinline__ void v_to_f32(const uint4& v, float (&out)[Geo<KV, D>::kEpl]) {
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (KV == PKV_F16) {
            out[2 * i] = f16_lo(vw[i]);
            out[2 * i + 1] = f16_hi(vw[i]);
        } else if constexpr (KV == PKV_BF16) {
            out[2 * i] = bf16_lo(vw[i]);
            out[2 * i + 1] = bf16_hi(vw[i]);
        } else {
            const float2_t lo = e4m3x2_lo(vw[i]);
            const float2_t hi = e4m3x2_hi(vw[i]);
            out[4 * i + 0] = lo.x;
            out[4 * i + 1] = lo.y;
            out[4 * i + 2] = hi.x;
            out[4 * i + 3] = hi.y;
        }
    }
}

template <int KV, int D>
struct Tile {
    uint4 k[Geo<KV, D>::kNld];
    uint4 v[Geo<KV, D>::kNld];
};

template <int KV, int D, int G>
struct SoftmaxState {
    float m[G];                       // running max, base-2 units
    float l[G];                       // running sum of exp2(s - m)
    float o[G][Geo<KV, D>::kEpl];     // running sum of exp2(s - m) * v, this lane's dims
};

// Fold one tile into the lane's online-softmax state. The tile's attended
// tokens are [nlo, nvalid) (nvalid: the context ends; nlo: a sliding window
// starts). kPartial selects the masked form, needed only when that is not the
// whole tile (the last block of a context, the window's first block, or a
// tile outside the context): other tokens get score -inf and their V bytes,
// which may be stale or NaN, are replaced by zeros.
template <int KV, int D, int G, bool kPartial>
__device__ __forceinline__ void consume_tile(SoftmaxState<KV, D, G>& st, const Tile<KV, D>& t,
                                             int nvalid, int nlo,
                                             const QSlice<KV, D> (&qs)[G], float sscale,
                                             int row) {
    using Gm = Geo<KV, D>;
    constexpr int EPL = Gm::kEpl, LPT = Gm::kLpt, TPI = Gm::kTpi, NLD = Gm::kNld;
    float sc[G][NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h][i] = qk_partial<KV, D>(t.k[i], qs[h]);
#pragma unroll
    for (int i = 0; i < NLD; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h][i] = group_sum<LPT>(sc[h][i]) * sscale;
    bool valid[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i)
        valid[i] = !kPartial || ((i * TPI + row) < nvalid && (i * TPI + row) >= nlo);
    if constexpr (kPartial) {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
#pragma unroll
            for (int h = 0; h < G; ++h) sc[h][i] = valid[i] ? sc[h][i] : -INFINITY;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float mx = st.m[h];
#pragma unroll
        for (int i = 0; i < NLD; ++i) mx = fmaxf(mx, sc[h][i]);
        const float ms = (mx == -INFINITY) ? 0.0f : mx;
        const float alpha = fast_exp2(st.m[h] - ms);
        st.m[h] = mx;
        float lsum = st.l[h] * alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.o[h][e] *= alpha;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            sc[h][i] = fast_exp2(sc[h][i] - ms);
            lsum += sc[h][i];
        }
        st.l[h] = lsum;
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        float vf[EPL];
        v_to_f32<KV, D>(t.v[i], vf);
        if constexpr (kPartial) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) vf[e] = valid[i] ? vf[e] : 0.0f;  // stale bytes never enter
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) st.o[h][e] = fmaf(sc[h][i], vf[e], st.o[h][e]);
    }
}

// Store one lane's EPL consecutive results of query head qh (dims
// [d0, d0 + EPL)): fp32 into the workspace, or rounded to the q dtype into out.
template <int QD, int D, int EPL>
__device__ __forceinline__ void store_result(const DecodeParams& p, int s, int qh, int part,
                                             int d0, const float (&r)[EPL]) {
    if (p.blocks_per_part > 0) {
        const size_t slot = (static_cast<size_t>(s) * p.num_q_heads + qh) * p.num_parts + part;
        float4* dst = reinterpret_cast<float4*>(p.ws_o + slot * D + d0);
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e)
            dst[e] = make_float4(r[4 * e], r[4 * e + 1], r[4 * e + 2], r[4 * e + 3]);
    } else {
        const size_t o_idx = (static_cast<size_t>(s) * p.num_q_heads + qh) * D + d0;
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + o_idx);
#pragma unroll
        for (int e = 0; e < EPL / 8; ++e) {
            uint32_t wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = r[8 * e + 2 * i], b = r[8 * e + 2 * i + 1];
                const uint32_t lo = (QD == PKV_F16) ? f32_to_f16_bits(a) : f32_to_bf16_bits(a);
                const uint32_t hi = (QD == PKV_F16) ? f32_to_f16_bits(b) : f32_to_bf16_bits(b);
                wv[i] = lo | (hi << 16);
            }
            dst[e] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    }
}

// Fused append on an FP8 cache: the new token of sequence s (kv head g, the
// last position L - 1, offset off of block id) is folded into the lane's
// softmax state after the wave's tile ring has drained. Its K and V source
// rows (parked in lds, see NewSrc) are encoded exactly as kv_cache_append
// encodes them, the codes go to the token's slot, and the attention uses the
// decoded codes, so the result is the one over the stored bytes. Lane col
// (= lane mod LPT) owns dims col*EPL .. +EPL, as in the tile loads.
template <int QD, int D, int G>
__device__ __forceinline__ void fold_new_token_fp8(const DecodeParams& p,
                                                   SoftmaxState<PKV_FP8_E4M3, D, G>& st,
                                                   const QSlice<PKV_FP8_E4M3, D> (&qs)[G],
                                                   float sscale, const uint8_t* lds, int g,
                                                   int id, int off, int lane) {
    using Gm = Geo<PKV_FP8_E4M3, D>;
    constexpr int EPL = Gm::kEpl, LPT = Gm::kLpt, TB = Gm::kTileBytes;
    static_assert(EPL == 16, "one lane holds 16 codes: two 8-element source chunks");
    const int col = lane % LPT;
    const float ks = p.k_scale[g], vs = p.v_scale[g];
    const uint2 k0 = quant_e4m3x8<QD>(new_chunk(lds, 0, 2 * col), ks);
    const uint2 k1 = quant_e4m3x8<QD>(new_chunk(lds, 0, 2 * col + 1), ks);
    const uint2 v0 = quant_e4m3x8<QD>(new_chunk(lds, 1, 2 * col), vs);
    const uint2 v1 = quant_e4m3x8<QD>(new_chunk(lds, 1, 2 * col + 1), vs);
    const uint4 kcode = make_uint4(k0.x, k0.y, k1.x, k1.y);
    const uint4 vcode = make_uint4(v0.x, v0.y, v1.x, v1.y);
    float kf[EPL], vf[EPL];
    v_to_f32<PKV_FP8_E4M3, D>(kcode, kf);
    v_to_f32<PKV_FP8_E4M3, D>(vcode, vf);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) part = fmaf(kf[e], qs[h].f[e], part);
        const float sn = group_sum<LPT>(part) * sscale;
        const float mx = fmaxf(st.m[h], sn);
        const float a = fast_exp2(st.m[h] - mx), b = fast_exp2(sn - mx);
        st.l[h] = st.l[h] * a + b;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.o[h][e] = fmaf(b, vf[e], st.o[h][e] * a);
        st.m[h] = mx;
    }
    if (lane < LPT) {
        const size_t at = (static_cast<size_t>(id) * p.num_kv_heads + g) * TB +
                          static_cast<size_t>(off) * D + col * 16;
        *reinterpret_cast<uint4*>(const_cast<uint8_t*>(p.k_plane) + at) = kcode;
        *reinterpret_cast<uint4*>(const_cast<uint8_t*>(p.v_plane) + at) = vcode;
    }
}

// Vector-ALU decode: one workgroup of NW wave64s per (kv head, sequence,
// partition). Each wave streams its tiles through a ring of NBUF tiles held in
// registers: after a tile is folded into the softmax state its registers are
// refilled with the tile NBUF positions ahead, so every wave keeps NBUF tiles
// of loads in flight from its first tile to its last. Used for FP8 caches and
// for one query head per kv head.
// kFused: the call also stores each sequence's new token, taken from the
// source rows (NewSrc). On 16-bit caches the wave reading the token's tile
// patches the row into the tile inside the ring. On FP8 caches that wave
// attends over the positions before the token, and the first wave of the
// workgroup that reads the context's first attended block (dispatched early,
// so its extra work stays off the kernel's tail) folds the token in after its
// ring has drained and stores it (fold_new_token_fp8); with split-K the token
// thus counts in that first partition's partial.
// kLds: the tile ring lives in LDS (two tiles per wave), filled by direct
// buffer-to-LDS loads, and a tile is read into registers only when it is
// consumed; otherwise (the default) the ring is NBUF tiles of registers.
template <int KV, int QD, int D, int G, int NW, int NBUF, bool kFused = false, bool kLds = false>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeParams p) {
    static_assert(!kLds || NBUF == 2, "LDS ring: two slots");
    constexpr bool kPatch = kFused && KV != PKV_FP8_E4M3;
    constexpr bool kFold = kFused && KV == PKV_FP8_E4M3;
    using Gm = Geo<KV, D>;
    constexpr int EPL = Gm::kEpl, LPT = Gm::kLpt, NLD = Gm::kNld, TB = Gm::kTileBytes;

    const int g = blockIdx.x;
    const int part = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int w = (NW == 1) ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane / LPT;
    const int col = lane % LPT;

    WaveWork ww;
    if (!locate_work<G, D, NW, kFused>(p, g, part, w, ww)) return;
    const int s = ww.s, L = ww.L, n = ww.n;
    BlockIds<NW> ids;
    ids.init(p.block_tables + static_cast<size_t>(s) * p.max_blocks + ww.b0, n, lane);

    // Query slices of the G heads of this group.
    QSlice<KV, D> qs[G];
    const uint16_t* qbase = static_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const size_t qrow = (static_cast<size_t>(s) * p.num_q_heads + g * G + h) * D;
        load_q<KV, QD, D>(qs[h], qbase + qrow, col);
    }
    float sscale = p.scale_log2;
    if constexpr (KV == PKV_FP8_E4M3) sscale *= p.k_scale[g];

    SoftmaxState<KV, D, G> st;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        st.m[h] = -INFINITY;
        st.l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.o[h][e] = 0.0f;
    }

    const uint8_t* kpl = p.k_plane + static_cast<size_t>(g) * TB;
    const uint8_t* vpl = p.v_plane + static_cast<size_t>(g) * TB;
    const size_t bstride = static_cast<size_t>(p.num_kv_heads) * TB;
    const int voff = lane * 16;

    Tile<KV, D> t[kLds ? 1 : NBUF];
    int nv[NBUF], nl[NBUF];
    // LDS ring: one array per slot, so that reading a slot waits only for
    // that slot's loads (the later slot's stay in flight).
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kLds ? NW : 1][kLds ? 2 * TB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kLds ? NW : 1][kLds ? 2 * TB : 16];
    // Fused append: the wave that reads the new token's tile fetches its
    // source rows first and parks them in LDS once they land (by then the
    // ring's first tiles are in flight behind them).
    __shared__ __attribute__((aligned(16))) uint8_t new_rows[kFused ? NW : 1][kFused ? 512 : 16];
    NewSrc<D> ns;
    // kPatch: the wave reading the new token's tile takes its rows; kFold: the
    // folding wave does, with the block id of the token's slot from the table.
    const bool takes_new = kPatch ? ww.newk >= 0 : (kFold && ww.fold);
    if (kFused && takes_new) ns.fetch(p, s, g, lane);
    int new_id = -1;
    if constexpr (kFold) {
        if (ww.fold)
            new_id = p.block_tables[static_cast<size_t>(s) * p.max_blocks + ((L - 1) >> 4)];
    }
    // Issue the loads of tile kn into a ring slot (x: the slot, for the LDS ring).
    auto issue = [&](Tile<KV, D>& tt, int& nvalid, int& nlo, int kn, int x) {
        const int id = ids.next(kn);
        // FP8 fused append: the new token (position L - 1) is folded in after
        // the ring, so its tile attends over the positions before it.
        const TileRef r = tile_ref(p, kpl, vpl, bstride, TB, id, (ww.b0 + kn * NW) * 16,
                                   (kFold && kn == ww.newk) ? L - 1 : L, ww.lo);
        nvalid = r.nvalid;
        nlo = r.nlo;  // > 0 only on a sliding window's first tile
        if (kPatch && kn == ww.newk) new_id = id;
        if constexpr (kLds) {
            typedef __attribute__((address_space(3))) void* lds_ptr;
            uint8_t* slot = x == 0 ? ring0[w] : ring1[w];
            // The slot's earlier reads must have completed: the refill's LDS
            // writes do not queue behind this wave's own LDS reads.
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
#pragma unroll
            for (int i = 0; i < NLD; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r.k, (lds_ptr)(slot + i * 1024), 16,
                                                         voff + i * 1024, 0, 0, kStreamPolicy);
#pragma unroll
            for (int i = 0; i < NLD; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r.v, (lds_ptr)(slot + TB + i * 1024), 16,
                                                         voff + i * 1024, 0, 0, kStreamPolicy);
        } else {
#pragma unroll
            for (int i = 0; i < NLD; ++i) tt.k[i] = rsrc_load16(r.k, voff + i * 1024);
#pragma unroll
            for (int i = 0; i < NLD; ++i) tt.v[i] = rsrc_load16(r.v, voff + i * 1024);
        }
    };

#pragma unroll
    for (int x = 0; x < NBUF; ++x) issue(t[kLds ? 0 : x], nv[x], nl[x], x, x);
    if (kFused && takes_new) ns.stash(new_rows[w], lane);
    for (int k0 = 0; k0 < n; k0 += NBUF) {
#pragma unroll
        for (int x = 0; x < NBUF; ++x) {
            Tile<KV, D>& tx = t[kLds ? 0 : x];
            if constexpr (kLds) {
                const uint8_t* slot = x == 0 ? ring0[w] : ring1[w];
                // Wait for this slot's loads (the other slot's 2*NLD stay in
                // flight) explicitly: the compiler's own wait for buffer-to-LDS
                // loads missed a read it had split and hoisted.
                static_assert(2 * NLD < 16, "vmcnt field");
                __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * NLD));  // vmcnt(2*NLD)
#pragma unroll
                for (int i = 0; i < NLD; ++i)
                    tx.k[i] = *reinterpret_cast<const uint4*>(slot + i * 1024 + voff);
#pragma unroll
                for (int i = 0; i < NLD; ++i)
                    tx.v[i] = *reinterpret_cast<const uint4*>(slot + TB + i * 1024 + voff);
            }
            if (kPatch && k0 + x == ww.newk && nv[x] > 0) {
                // The new token (the last of the context): from the source
                // rows into the tile and into its slot.
                const int off = nv[x] - 1;
                const uint4 kc = new_chunk(new_rows[w], 0, col);
                const uint4 vc = new_chunk(new_rows[w], 1, col);
                patch_natural<LPT>(tx.k, kc, off, lane);
                patch_natural<LPT>(tx.v, vc, off, lane);
                store_new_row<LPT>(p, g, new_id, off, TB, kc, vc, lane);
            }
            // LDS ring: the tile is in registers now, so the slot is refilled
            // before the math (two tiles stay in flight while it runs).
            const int cnv = nv[x], cnl = nl[x];
            if constexpr (kLds) issue(tx, nv[x], nl[x], k0 + x + NBUF, x);
            if (cnv == 16 && cnl == 0)
                consume_tile<KV, D, G, false>(st, tx, 16, 0, qs, sscale, row);
            else
                consume_tile<KV, D, G, true>(st, tx, cnv, cnl, qs, sscale, row);
            if constexpr (!kLds) issue(tx, nv[x], nl[x], k0 + x + NBUF, x);
        }
    }

    // Merge the rows of this wave: lanes lane ^ off (off = LPT, 2*LPT, ...)
    // hold the same dims for other tokens.
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m2 = __shfl_xor(st.m[h], off);
            const float l2 = __shfl_xor(st.l[h], off);
            const float mx = fmaxf(st.m[h], m2);
            const float ms = (mx == -INFINITY) ? 0.0f : mx;
            const float a = fast_exp2(st.m[h] - ms), b = fast_exp2(m2 - ms);
            st.l[h] = st.l[h] * a + l2 * b;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float o2 = __shfl_xor(st.o[h][e], off);
                st.o[h][e] = st.o[h][e] * a + o2 * b;
            }
            st.m[h] = mx;
        }
    }

    if constexpr (kFold) {
        if (ww.fold && static_cast<uint32_t>(new_id) < static_cast<uint32_t>(p.num_blocks))
            fold_new_token_fp8<QD, D, G>(p, st, qs, sscale, new_rows[w], g, new_id, (L - 1) & 15,
                                         lane);
    }

    float vscale = 1.0f;
    if constexpr (KV == PKV_FP8_E4M3) vscale = p.v_scale[g];

    if constexpr (NW == 1) {
        if (row == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float inv = st.l[h] > 0.0f ? vscale / st.l[h] : 0.0f;
                float r[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) r[e] = st.o[h][e] * inv;
                store_result<QD, D, EPL>(p, s, g * G + h, part, col * EPL, r);
                if (p.blocks_per_part > 0 && col == 0) store_ml(p, s, g * G + h, part, st.m[h], st.l[h]);
            }
        }
    } else {
        // Merge the NW waves through LDS.
        __shared__ float lds_o[NW][G][D];
        __shared__ float lds_m[NW][G];
        __shared__ float lds_l[NW][G];
        if (row == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < EPL; ++e) lds_o[w][h][col * EPL + e] = st.o[h][e];
        }
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                lds_m[w][h] = st.m[h];
                lds_l[w][h] = st.l[h];
            }
        }
        __syncthreads();
        combine_waves<QD, D, G, NW>(p, s, g, part, lds_o, lds_m, lds_l, vscale);
    }
}

}  // namespace
