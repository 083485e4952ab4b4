// Gather-rate probe: the paged decode's memory access pattern with no
// arithmetic, to measure the rate at which one MI355X delivers scattered
// 16 x D tiles (K from one plane, V from another) to its waves. It is a
// measuring instrument for the decode kernels' roofline, not part of the
// decode path, and lives in a library of its own (libpkvprobe.so).
//
// Each wave streams its list of tile ids; tile t is the 4 KiB K tile at
// k_plane + id * 4096 and the V tile at the same offset of v_plane, read with
// 16-byte non-temporal buffer loads like the decode's. Staging forms:
//  * mode 0: a ring of three tiles held in registers (the decode kernels'
//    form): a consumed tile's registers are refilled at once with the tile
//    three ahead;
//  * mode 1 / 2: a ring of two / three tiles in LDS, filled by direct
//    buffer-to-LDS loads (no registers held for tiles in flight) and read
//    back with ds_read_b128 when consumed.
// Consuming a tile XORs its words into a per-lane value that is stored only
// if it hits a sentinel, so no load is optimised away.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kTile = 4096;  // bytes of one K (or V) tile: 16 tokens x 128 dims x 2 bytes
constexpr int kLoads = kTile / 1024;  // 16-byte loads per lane per tile

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* plane, int id,
                                                           int num_tiles) {
    const bool ok = static_cast<uint32_t>(id) < static_cast<uint32_t>(num_tiles);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(plane) + static_cast<size_t>(ok ? id : 0) * kTile,
        static_cast<short>(0), ok ? kTile : 0, 0x00020000);
}

__device__ __forceinline__ uint32_t fold(const uint4& x) { return x.x ^ x.y ^ x.z ^ x.w; }

struct RegTile {
    uint4 k[kLoads], v[kLoads];
};

template <int W>
__global__ __launch_bounds__(W * 64) void gather_regs(const uint8_t* kp, const uint8_t* vp,
                                                     const int32_t* ids, int per_wave,
                                                     int num_tiles, uint32_t* sink) {
    constexpr int R = 3;
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * W + (threadIdx.x >> 6);
    // the wave's ids (at most 64) in one vector load, broadcast with readlane
    const int my_ids = lane < per_wave ? ids[static_cast<size_t>(wave) * per_wave + lane] : -1;
    uint32_t acc = 0;
    RegTile t[R];
    auto issue = [&](RegTile& tt, int k) {
        const int id = k < per_wave ? __builtin_amdgcn_readlane(my_ids, k) : -1;
        const auto rk = tile_rsrc(kp, id, num_tiles), rv = tile_rsrc(vp, id, num_tiles);
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            tt.k[i] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, lane * 16 + i * 1024, 0, 2));
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            tt.v[i] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane * 16 + i * 1024, 0, 2));
    };
#pragma unroll
    for (int x = 0; x < R; ++x) issue(t[x], x);
    for (int k0 = 0; k0 < per_wave; k0 += R) {
#pragma unroll
        for (int x = 0; x < R; ++x) {
#pragma unroll
            for (int i = 0; i < kLoads; ++i) acc ^= fold(t[x].k[i]) ^ fold(t[x].v[i]);
            issue(t[x], k0 + x + R);
        }
    }
    if (acc == 0x9E3779B9u) sink[static_cast<size_t>(wave) * 64 + lane] = acc;
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// One ring slot in LDS per array: distinct arrays let the compiler wait for
// exactly the slot being read (vmcnt of the later slots' loads), not for all.
template <int W, int R>
__global__ __launch_bounds__(W * 64) void gather_lds(const uint8_t* kp, const uint8_t* vp,
                                                    const int32_t* ids, int per_wave,
                                                    int num_tiles, uint32_t* sink) {
    static_assert(R == 2 || R == 3, "ring depth");
    __shared__ __attribute__((aligned(16))) uint8_t s0[W][2 * kTile];
    __shared__ __attribute__((aligned(16))) uint8_t s1[W][2 * kTile];
    __shared__ __attribute__((aligned(16))) uint8_t s2[R == 3 ? W : 1][R == 3 ? 2 * kTile : 16];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave = blockIdx.x * W + w;
    const int my_ids = lane < per_wave ? ids[static_cast<size_t>(wave) * per_wave + lane] : -1;
    uint32_t acc = 0;
    auto issue = [&](uint8_t* slot, int k) {
        const int id = k < per_wave ? __builtin_amdgcn_readlane(my_ids, k) : -1;
        const auto rk = tile_rsrc(kp, id, num_tiles), rv = tile_rsrc(vp, id, num_tiles);
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)(slot + i * 1024), 16,
                                                     lane * 16 + i * 1024, 0, 0, 2);
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)(slot + kTile + i * 1024), 16,
                                                     lane * 16 + i * 1024, 0, 0, 2);
    };
    auto consume = [&](const uint8_t* slot) {
        uint32_t a = 0;
#pragma unroll
        for (int i = 0; i < 2 * kLoads; ++i)
            a ^= fold(reinterpret_cast<const uint4*>(slot + i * 1024)[lane]);
        acc ^= a;
        // the slot's reads complete before its refill is issued
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt and expcnt untouched
    };
    issue(s0[w], 0);
    issue(s1[w], 1);
    if constexpr (R == 3) issue(s2[w], 2);
    for (int k0 = 0; k0 < per_wave; k0 += R) {
        consume(s0[w]);
        issue(s0[w], k0 + R);
        consume(s1[w]);
        issue(s1[w], k0 + R + 1);
        if constexpr (R == 3) {
            consume(s2[w]);
            issue(s2[w], k0 + R + 2);
        }
    }
    if (acc == 0x9E3779B9u) sink[static_cast<size_t>(wave) * 64 + lane] = acc;
}

}  // namespace

// Launch one probe pass: num_waves waves of waves_per_wg per workgroup, wave w
// streaming ids[w * per_wave .. + per_wave), per_wave <= 64 (ids outside
// [0, num_tiles) read nothing). k_plane, v_plane: device buffers of num_tiles * 4096 bytes each;
// sink: device uint32 [num_waves * 64]. mode 0: register ring of three tiles;
// 1: LDS ring of two; 2: LDS ring of three. Returns a hipError_t code.
extern "C" __attribute__((visibility("default"))) int pkv_probe_gather(
    const void* k_plane, const void* v_plane, const int32_t* ids, int32_t num_waves,
    int32_t per_wave, int32_t num_tiles, int32_t mode, int32_t waves_per_wg, uint32_t* sink,
    hipStream_t stream) {
    if (k_plane == nullptr || v_plane == nullptr || ids == nullptr || sink == nullptr ||
        num_waves <= 0 || per_wave <= 0 || per_wave > 64 || num_tiles <= 0 || num_waves % waves_per_wg != 0 ||
        (waves_per_wg != 1 && waves_per_wg != 2 && waves_per_wg != 4) || mode < 0 || mode > 2)
        return static_cast<int>(hipErrorInvalidValue);
    const dim3 grid(static_cast<uint32_t>(num_waves / waves_per_wg));
    const auto* kp = static_cast<const uint8_t*>(k_plane);
    const auto* vp = static_cast<const uint8_t*>(v_plane);
#define PKV_PROBE_LAUNCH(KERNEL, WV)                                                          \
    hipLaunchKernelGGL((KERNEL), grid, dim3((WV) * 64), 0, stream, kp, vp, ids, per_wave, \
                       num_tiles, sink)
    switch (mode * 8 + waves_per_wg) {
        case 0 * 8 + 1: PKV_PROBE_LAUNCH((gather_regs<1>), 1); break;
        case 0 * 8 + 2: PKV_PROBE_LAUNCH((gather_regs<2>), 2); break;
        case 0 * 8 + 4: PKV_PROBE_LAUNCH((gather_regs<4>), 4); break;
        case 1 * 8 + 1: PKV_PROBE_LAUNCH((gather_lds<1, 2>), 1); break;
        case 1 * 8 + 2: PKV_PROBE_LAUNCH((gather_lds<2, 2>), 2); break;
        case 1 * 8 + 4: PKV_PROBE_LAUNCH((gather_lds<4, 2>), 4); break;
        case 2 * 8 + 1: PKV_PROBE_LAUNCH((gather_lds<1, 3>), 1); break;
        case 2 * 8 + 2: PKV_PROBE_LAUNCH((gather_lds<2, 3>), 2); break;
        default: PKV_PROBE_LAUNCH((gather_lds<4, 3>), 4); break;
    }
#undef PKV_PROBE_LAUNCH
    return static_cast<int>(hipGetLastError());
}
