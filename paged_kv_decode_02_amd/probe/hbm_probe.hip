// HBM read-throughput probe for the decode kernels' access pattern (a
// measurement aid, not part of libpa): every wave streams a run of random
// 4 KB (page, kv-head) tiles of two pools (K and V), TPB tiles of each per
// batch (2 or 4), the next batch's loads issued before the current one is
// consumed -- the pipeline the stream kernels use -- by one of two load
// paths:
//  * mode 0: global_load_lds_dwordx4 (16 bytes per lane straight into LDS,
//    1 KB per instruction), waited for by vmcnt, as the stream kernels do;
//  * mode 1: global_load_dwordx4 into registers, 32 KB per batch per wave,
//    folded into a checksum so that no load is dead.
// Bytes read per launch = tiles * 4 KB * 2; the host reports them over the
// kernel time (HIP events).  C ABI: hbm_probe_run.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kTile = 4096;
constexpr int kLoadsPerTile = kTile / 1024;  // 1 KB per wave-wide 16-byte load

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<size_t>((__attribute__((address_space(3))) const void*)(p)));
}

__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_base) : "memory");
}

// One wave per workgroup; wave w streams tiles [w * per, (w + 1) * per) of
// `ids` (tile indices into both pools, in [0, n_tiles)).
template <int MODE, int TPB>
__global__ __launch_bounds__(64) void probe_kernel(const char* __restrict__ kpool, const char* __restrict__ vpool,
                                                   const int32_t* __restrict__ ids, int per, int total,
                                                   uint32_t* __restrict__ sink) {
  constexpr int NL = TPB * kLoadsPerTile;  // 1 KB loads per pool per batch
  __shared__ uint4 lds[MODE == 0 ? 2 : 1][2][MODE == 0 ? NL * 64 : 1];  // [buffer][K, V][TPB tiles]
  const int lane = threadIdx.x;
  const int a = blockIdx.x * per;
  const int b = min(a + per, total);
  if (a >= b) return;
  const int nb = (b - a + TPB - 1) / TPB;  // batches of TPB tiles
  uint32_t acc = 0;
  auto tile_of = [&](int bt, int i) { return ids[min(a + TPB * bt + i, b - 1)]; };
  if constexpr (MODE == 0) {
    auto issue = [&](int bt, int buf) {
#pragma unroll
      for (int i = 0; i < TPB; ++i) {
        const int64_t t = tile_of(bt, i);
#pragma unroll
        for (int j = 0; j < kLoadsPerTile; ++j) {
          dma16(kpool + t * kTile + j * 1024 + lane * 16, lds_addr(&lds[buf][0][(i * kLoadsPerTile + j) * 64]));
          dma16(vpool + t * kTile + j * 1024 + lane * 16, lds_addr(&lds[buf][1][(i * kLoadsPerTile + j) * 64]));
        }
      }
    };
    issue(0, 0);
    for (int bt = 0; bt < nb; ++bt) {
      const int buf = bt & 1;
      if (bt + 1 < nb) {
        issue(bt + 1, buf ^ 1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL) : "memory");  // this batch's 2 NL loads done
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
      // consume one dword per lane of each KB so the loads are used
#pragma unroll
      for (int j = 0; j < NL; ++j) acc ^= lds[buf][0][j * 64 + lane].x ^ lds[buf][1][j * 64 + lane].y;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  } else {
    uint4 cur[2][NL], nxt[2][NL];
    auto load = [&](int bt, uint4 (&dst)[2][NL]) {
#pragma unroll
      for (int i = 0; i < TPB; ++i) {
        const int64_t t = tile_of(bt, i);
#pragma unroll
        for (int j = 0; j < kLoadsPerTile; ++j) {
          dst[0][i * kLoadsPerTile + j] = *reinterpret_cast<const uint4*>(kpool + t * kTile + j * 1024 + lane * 16);
          dst[1][i * kLoadsPerTile + j] = *reinterpret_cast<const uint4*>(vpool + t * kTile + j * 1024 + lane * 16);
        }
      }
    };
    load(0, cur);
    for (int bt = 0; bt < nb; ++bt) {
      if (bt + 1 < nb) load(bt + 1, nxt);
#pragma unroll
      for (int j = 0; j < NL; ++j)
        acc ^= cur[0][j].x ^ cur[0][j].y ^ cur[0][j].z ^ cur[0][j].w ^ cur[1][j].x ^ cur[1][j].y ^ cur[1][j].z ^
               cur[1][j].w;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        cur[0][j] = nxt[0][j];
        cur[1][j] = nxt[1][j];
      }
    }
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;  // (practically never; keeps acc live)
}

}  // namespace

// Runs the probe `reps` times with `waves` waves (one per workgroup) over
// `total` tile ids (device array, each in [0, n_tiles) of both pools, which
// hold n_tiles * 4 KB each), `tpb` (2 or 4) tiles of each pool per batch;
// returns the mean kernel time in ms, or a negative value on an error.
extern "C" float hbm_probe_run(int mode, int tpb, const void* kpool, const void* vpool, const int32_t* ids,
                               int total, int waves, int reps, void* stream) {
  if (waves < 1 || total < 1 || reps < 1 || !kpool || !vpool || !ids || (mode != 0 && mode != 1) ||
      (tpb != 2 && tpb != 4))
    return -1.f;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int per = (total + waves - 1) / waves;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -2.f;
  auto launch = [&]() {
    auto k = mode == 0 ? (tpb == 2 ? probe_kernel<0, 2> : probe_kernel<0, 4>)
                       : (tpb == 2 ? probe_kernel<1, 2> : probe_kernel<1, 4>);
    hipLaunchKernelGGL(k, dim3(waves), dim3(64), 0, st, static_cast<const char*>(kpool),
                       static_cast<const char*>(vpool), ids, per, total, static_cast<uint32_t*>(nullptr));
  };
  launch();  // warm-up
  (void)hipEventRecord(e0, st);
  for (int r = 0; r < reps; ++r) launch();
  (void)hipEventRecord(e1, st);
  float ms = -3.f;
  if (hipEventSynchronize(e1) == hipSuccess && hipGetLastError() == hipSuccess) {
    (void)hipEventElapsedTime(&ms, e0, e1);
    ms /= reps;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return ms;
}
