// HBM stream probes: the practical bandwidth ceilings of the access mixes
// the library's kernels use, measured with kernels that do nothing but move
// bytes.  Built as a library of its own (libla_probes.so), used only by the
// benchmark; it is not part of the attention path.
//
//   read   : 16-byte loads, the values folded into a register (the mix of the
//            KV reduction, which only reads)
//   write  : 16-byte stores of a constant
//   copy   : 16-byte loads and stores, one read byte per written byte
//   widen  : bfloat16 in, float32 out: one read byte per two written bytes
//            (the readout's mix: bf16 queries in, float32 rows out).  Every
//            store instruction of a wavefront writes 1 KB contiguously, as the
//            readout's stores do.
//
// Schedules (how a workgroup's steps map onto memory):
//   sweep   : a persistent grid of G workgroups; step j of workgroup w takes
//             chunk j G + w, so the whole grid walks one window of memory
//   range   : a persistent grid; workgroup w takes one contiguous range
//   oneshot : one workgroup per chunk (grid = number of chunks)
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kU = 4;  // 16-byte units per thread per step (read, write, copy)
constexpr int kWU = 2; // 1 KB wave blocks per wave per step (widen)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Mode { kRead = 0, kWrite = 1, kCopy = 2, kWiden = 3 };
enum Sched { kSweep = 0, kRange = 1, kOneshot = 2 };

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}
template <bool NT>
__device__ __forceinline__ u32x2 ld8(const u32x2* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}
template <bool NT>
__device__ __forceinline__ void st16(u32x4* p, u32x4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// One step of chunk c.  A chunk is kThreads * kU 16-byte units of the read
// side (read, copy), of the written side (write), or 4 waves * kWU wave
// blocks of 512 elements (widen).
template <int MODE, bool NTL, bool NTS>
__device__ __forceinline__ void step(const void* src, void* dst, long long c, u32x4& acc) {
  const int tid = threadIdx.x;
  if constexpr (MODE == kWiden) {
    const int lane = tid & 63, wave = tid >> 6;
    const uint16_t* in = static_cast<const uint16_t*>(src);
    float* out = static_cast<float*>(dst);
    u32x2 x[kWU][2];
#pragma unroll
    for (int b = 0; b < kWU; ++b) {
      const long long base = ((c * 4 + wave) * kWU + b) * 512;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        x[b][h] = ld8<NTL>(reinterpret_cast<const u32x2*>(in + base + 256 * h + 4 * lane));
    }
#pragma unroll
    for (int b = 0; b < kWU; ++b) {
      const long long base = ((c * 4 + wave) * kWU + b) * 512;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 y = {x[b][h].x << 16, x[b][h].x & 0xFFFF0000u, x[b][h].y << 16,
                         x[b][h].y & 0xFFFF0000u};
        st16<NTS>(reinterpret_cast<u32x4*>(out + base + 256 * h + 4 * lane), y);
      }
    }
  } else {
    const u32x4* in = static_cast<const u32x4*>(src);
    u32x4* out = static_cast<u32x4*>(dst);
    const long long base = c * (kThreads * kU) + tid;
    u32x4 v[kU];
    if constexpr (MODE != kWrite) {
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = ld16<NTL>(in + base + kThreads * u);
    }
    if constexpr (MODE == kRead) {
#pragma unroll
      for (int u = 0; u < kU; ++u) acc ^= v[u];
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const u32x4 y = MODE == kWrite ? acc : v[u];
        st16<NTS>(out + base + kThreads * u, y);
      }
    }
  }
}

template <int MODE, int SCHED, bool NTL, bool NTS>
__global__ __launch_bounds__(kThreads) void stream_probe(const void* src, void* dst,
                                                         long long nchunks, uint32_t magic,
                                                         u32x4* sink) {
  u32x4 acc = {threadIdx.x, blockIdx.x, 0u, 1u};
  const long long G = gridDim.x, w = blockIdx.x;
  if constexpr (SCHED == kOneshot) {
    if (w < nchunks) step<MODE, NTL, NTS>(src, dst, w, acc);
  } else if constexpr (SCHED == kSweep) {
    for (long long c = w; c < nchunks; c += G) step<MODE, NTL, NTS>(src, dst, c, acc);
  } else {
    const long long c0 = nchunks * w / G, c1 = nchunks * (w + 1) / G;
    for (long long c = c0; c < c1; ++c) step<MODE, NTL, NTS>(src, dst, c, acc);
  }
  // keeps the loads of the read probe alive; magic never matches in practice
  if constexpr (MODE == kRead)
    if (acc.x == magic && acc.y == magic && acc.z == magic && acc.w == magic)
      sink[threadIdx.x] = acc;
}

template <int MODE, int SCHED, bool NTL, bool NTS>
int launch(const void* src, void* dst, long long nchunks, int wgs, u32x4* sink,
           hipStream_t stream) {
  const long long grid = SCHED == kOneshot ? nchunks : wgs;
  if (grid <= 0 || grid > 0x7FFFFFFF) return 1;
  stream_probe<MODE, SCHED, NTL, NTS><<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(
      src, dst, nchunks, 0xFFFFFFFFu, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

template <int MODE, int SCHED>
int launch_nt(const void* src, void* dst, long long nchunks, int wgs, int ntl, int nts,
              u32x4* sink, hipStream_t stream) {
  if (ntl && nts) return launch<MODE, SCHED, true, true>(src, dst, nchunks, wgs, sink, stream);
  if (ntl) return launch<MODE, SCHED, true, false>(src, dst, nchunks, wgs, sink, stream);
  if (nts) return launch<MODE, SCHED, false, true>(src, dst, nchunks, wgs, sink, stream);
  return launch<MODE, SCHED, false, false>(src, dst, nchunks, wgs, sink, stream);
}

template <int MODE>
int launch_sched(const void* src, void* dst, long long nchunks, int wgs, int sched, int ntl,
                 int nts, u32x4* sink, hipStream_t stream) {
  switch (sched) {
    case kSweep: return launch_nt<MODE, kSweep>(src, dst, nchunks, wgs, ntl, nts, sink, stream);
    case kRange: return launch_nt<MODE, kRange>(src, dst, nchunks, wgs, ntl, nts, sink, stream);
    case kOneshot:
      return launch_nt<MODE, kOneshot>(src, dst, nchunks, wgs, ntl, nts, sink, stream);
    default: return 1;
  }
}

}  // namespace

extern "C" {

// Bytes one chunk of `mode` reads and writes.
int lap_chunk_bytes(int mode, long long* read_bytes, long long* write_bytes) {
  const long long units = static_cast<long long>(kThreads) * kU * 16;
  switch (mode) {
    case kRead: *read_bytes = units; *write_bytes = 0; return 0;
    case kWrite: *read_bytes = 0; *write_bytes = units; return 0;
    case kCopy: *read_bytes = units; *write_bytes = units; return 0;
    case kWiden:
      *read_bytes = 4LL * kWU * 512 * 2;
      *write_bytes = 4LL * kWU * 512 * 4;
      return 0;
    default: return 1;
  }
}

// One probe launch over `nchunks` chunks on `stream`.  src and dst are
// device buffers of at least nchunks times the chunk's read and written
// bytes (lap_chunk_bytes), 16-byte aligned; sink is a device buffer of 4 KB
// that the read probe could write (it never does for real data).  Returns 0,
// 1 for bad arguments, 2 for a launch failure.
int lap_stream(int mode, int sched, int wgs, int nt_loads, int nt_stores, const void* src,
               void* dst, long long nchunks, void* sink, hipStream_t stream) {
  if (nchunks <= 0 || (sched != kOneshot && wgs <= 0)) return 1;
  if ((mode != kWrite && src == nullptr) || (mode != kRead && dst == nullptr) ||
      sink == nullptr)
    return 1;
  u32x4* s = static_cast<u32x4*>(sink);
  switch (mode) {
    case kRead: return launch_sched<kRead>(src, dst, nchunks, wgs, sched, nt_loads, 0, s, stream);
    case kWrite:
      return launch_sched<kWrite>(src, dst, nchunks, wgs, sched, 0, nt_stores, s, stream);
    case kCopy:
      return launch_sched<kCopy>(src, dst, nchunks, wgs, sched, nt_loads, nt_stores, s, stream);
    case kWiden:
      return launch_sched<kWiden>(src, dst, nchunks, wgs, sched, nt_loads, nt_stores, s, stream);
    default: return 1;
  }
}

}  // extern "C"
