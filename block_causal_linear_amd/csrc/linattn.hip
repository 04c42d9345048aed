// Host side of the C ABI declared in include/linattn.h: argument checks,
// launch planning, and the three launches of a forward call (KV reduction ->
// split reduce + state add, or the prefix over blocks -> readout) or of a
// backward call (query gradients + partial state gradients -> suffix over
// blocks -> key and value gradients) on the caller's stream.  Nothing here
// allocates device memory or synchronises.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "linattn.h"
#include "la_common.h"
#include "kv_reduce.h"
#include "readout.h"
#include "state_update.h"
#include "backward.h"
#include "temporal_conv.h"
#include "rope.h"
#include "rope_bwd.h"

// Device scratch of the allocation-free backward entry point
// (la_blockcausal_backward_noalloc): a fixed array in the code object, one
// copy per GPU the library runs on, held until the process ends.  Host code
// never passes `scratch` itself to a kernel (on the host the name is only a
// stand-in for the symbol): it takes each device's address once, through
// hipGetSymbolAddress with that device current, and passes that pointer.
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kAbiVersion = 13;

// The address of `scratch` on the device of `stream` (the current device for
// the null stream), looked up on that device's first call and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return LA_E_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return LA_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return LA_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return LA_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return LA_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return LA_E_HIP;
    if (e != hipSuccess || p == nullptr) return LA_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LA_OK;
}

// A second stream of the library's own per device (default priority, created
// on the first backward call that can use it, kept until the process ends),
// with the two events that fork work onto it and join it back.  The backward
// runs the second half of its (b, h) pairs there (see backward()).
struct AuxStream {
  std::mutex mu;  // creation, then each call's fork / enqueue / join sequence
  bool tried = false;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
AuxStream g_aux[kMaxDevices];

AuxStream* aux_stream(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  AuxStream& a = g_aux[dev];
  std::lock_guard<std::mutex> lock(a.mu);
  if (!a.tried) {
    a.tried = true;  // a failed creation is not retried: calls stay on one stream
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    const bool ok = hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess &&
                    hipEventCreateWithFlags(&f, hipEventDisableTiming) == hipSuccess &&
                    hipEventCreateWithFlags(&j, hipEventDisableTiming) == hipSuccess;
    const bool back = cur == dev || hipSetDevice(cur) == hipSuccess;
    if (ok && back) {
      a.s = st;
      a.fork = f;
      a.join = j;
    }
  }
  return a.s != nullptr ? &a : nullptr;
}

// KV workgroups the planner aims for: two per compute unit of a 256-CU
// MI355X at d <= 64 (four waves each; measured best at the 720p chunk: 16
// splits x 32 heads), one per compute unit at d = 128 (sixteen waves each).
constexpr int kKvTargetWorkgroups = 512;
// The rotary KV kernel (bound by instruction issue, not bandwidth) gains from
// a third workgroup per CU at d <= 64: 134 us against 150 us at the 720p
// chunk (24 splits against 16).
constexpr int kKvRopeTargetWorkgroups = 768;
// A split should carry at least this many tokens per (d + 1) so that its
// partial (d*d + d floats) stays small next to the K/V bytes it reads.
constexpr int kKvMinTokensPerFeature = 4;
// Readout workgroups the planner aims for.  The sweep readout (bf16 inputs)
// runs three or four waves per SIMD at d <= 64: with its non-temporal stores
// 512 workgroups of four waves measured best at the 720p shape (171 us
// against 172-176 us for 768; 384 and 640 were slower).  The float32 readout
// gives each workgroup a contiguous token range of one head (1024
// workgroups, 512 at d = 128 where each stages a 64 KB state).
constexpr int kSweepWorkgroups = 512;
constexpr int kReadoutTargetWorkgroups = 1024;
// Shortest item of the item readout (d = 128): at the long-horizon chunk
// (64 heads x 4,096 tokens) items of 1,024 tokens on 256 workgroups measured
// 49.7 us against 54.1 us for 512-token items on 512 workgroups.
constexpr int kReadoutItemMinTokens = 1024;
// Compute units of an MI355X: the persistent grids below are sized to the
// resident workgroups of one round.
constexpr int kCUs = 256;
// One block at d = 128 takes the quadrant KV kernel (four workgroups per
// head, no token split) from this many (b, h) pairs: one workgroup per CU.
constexpr long long kKvQuadMinPairs = 64;
// Resident workgroups of the two bf16 backward kernels on a 256-CU MI355X:
// their persistent grids.  Each kernel is compiled for a number of waves
// per SIMD (its launch bound), which with four-wave workgroups is the
// number of workgroups per CU.
int bwd_query_capacity(int d) {
  return kCUs * (d == 128 ? la::bwd_query_min_waves<128>()
                 : d == 64 ? la::bwd_query_min_waves<64>()
                           : la::bwd_query_min_waves<32>());
}
int bwd_key_capacity(int d, bool rope) {
  if (rope)
    return kCUs * (d == 128 ? la::bwd_key_rope_min_waves<128>()
                   : d == 64 ? la::bwd_key_rope_min_waves<64>()
                             : la::bwd_key_rope_min_waves<32>());
  return kCUs * (d == 128 ? la::bwd_key_min_waves<128>()
                 : d == 64 ? la::bwd_key_min_waves<64>()
                           : la::bwd_key_min_waves<32>());
}
// Rotary calls: sequences (and frame offsets) below this many tokens.
constexpr int kRopeMaxTokens = 1 << 22;
// float32 backward kernels: workgroups over contiguous token ranges.
constexpr int kBwdF32TargetWorkgroups = 512;
// The key-gradient sweep (bf16, d <= 64, no rotary) and its grid: two
// workgroups per CU (64 KB of LDS each at d = 64).  Measured per call: the
// 720p chunk 664 us with 512 workgroups, 684 with 256, 703 with 384; the 480p
// stream in one call 1,693, 1,680 and 1,821 us.  LA_BWDK_SWEEP 0 keeps the
// work-item kernel for every call.
#ifndef LA_BWDK_SWEEP
#define LA_BWDK_SWEEP 1
#endif
#ifndef LA_BWDK_SWEEP_WGS
#define LA_BWDK_SWEEP_WGS 512
#endif
constexpr int kBwdKeySweepWorkgroups = LA_BWDK_SWEEP_WGS;
// Token-heads (B H N) from which a bfloat16 backward call runs its two halves
// of (b, h) pairs on two streams; below it the fork and join cost more than
// the overlap gains.
constexpr long long kBwdSplitMinTokens = 1LL << 20;

long long gcd_ll(long long a, long long b) {
  while (b != 0) {
    const long long t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Items per block for a persistent grid of `cap` workgroups over `pairs`
// (b, h, block) pairs: pairs * S = lcm(pairs, cap), a whole number of
// rounds of the grid, unless that needs more than about four rounds.
long long items_per_block(long long pairs, long long cap) {
  long long s = cap / gcd_ll(pairs, cap);
  const long long most = (4 * cap + pairs - 1) / pairs;
  return s < most ? s : most;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int elem_size(int dt) { return dt == LA_BF16 ? 2 : 4; }

struct Plan {
  int nblk;            // blocks of T tokens (0 when N == 0)
  int T;               // tokens per block (the last may be shorter)
  int splits;          // token splits per block for the KV reduction
  int tps;             // tokens per split
  int kv_tile;         // tokens per KV tile
  bool direct;         // one block, one split: the KV kernel writes the state
  bool quad;           // one block at d = 128: kv_quad_bf16 writes the state
  bool in_place;       // several blocks, one split: partials live in `states`
  bool sweep;          // readout_sweep_bf16 (bf16 inputs, d < LA_READOUT_ITEMS_MIN_D)
  bool items;          // readout_items_bf16 (bf16 inputs, larger d or rotary); else readout_f32
  int ro_splits;       // readout_items_bf16: items per block
  int readout_tpw;     // readout_f32: tokens per workgroup
  int readout_wgs;     // readout workgroups in the grid
  int units_per_block; // sweep readout: four-tile units per block
  int run_log2;        // sweep readout: log2 of the units per workgroup step
};

int check_shape(int B, int H, int N, int d, int in_dt, int out_dt) {
  if (B <= 0 || H <= 0 || N < 0) return LA_E_INVAL;
  if (B > 65535 || H > 65535) return LA_E_INVAL;
  if (d != 32 && d != 64 && d != 128) return LA_E_UNSUPPORTED;
  if ((in_dt != LA_F32 && in_dt != LA_BF16) || (out_dt != LA_F32 && out_dt != LA_BF16))
    return LA_E_UNSUPPORTED;
  // keep every per-head element index inside 31 bits
  if (static_cast<long long>(N) * d >= (1LL << 31)) return LA_E_INVAL;
  return LA_OK;
}

// Every tensor a call touches stays below 1 TiB, more than one GPU holds:
// byte counts, grid sizes and work-item counts then stay in range for any
// int arguments.  `factors` multiply to a byte count.
constexpr unsigned long long kMaxTensorBytes = 1ULL << 40;
bool bytes_below_limit(std::initializer_list<unsigned long long> factors) {
  for (unsigned long long f : factors)
    if (f == 0) return true;
  unsigned long long prod = 1;
  for (unsigned long long f : factors) {
    if (prod > (kMaxTensorBytes - 1) / f) return false;
    prod *= f;
  }
  return true;
}

// The token tensors ([B][H][N][d], at most 4 bytes an element) and the block
// states ([B][H][blocks][d*d + d] float32) of a call with blocks of T tokens.
int check_sizes(int B, int H, int N, int T, int d) {
  const int t = T < N ? T : N;
  const unsigned long long nblk = N == 0 ? 1 : (static_cast<unsigned long long>(N) + t - 1) / t;
  const unsigned long long st = (static_cast<unsigned long long>(d) * d + d) * sizeof(float);
  const unsigned long long b = static_cast<unsigned long long>(B);
  const unsigned long long h = static_cast<unsigned long long>(H);
  if (!bytes_below_limit({b, h, static_cast<unsigned long long>(N) * d, 4}) ||
      !bytes_below_limit({b, h, nblk, st}))
    return LA_E_INVAL;
  return LA_OK;
}

// N tokens per (b, h) in blocks of T (T >= N: one block).
// rope: the rotary readout runs on work items at every d.
Plan make_plan(int B, int H, int N, int T, int d, int in_dt, int out_dt, int request,
               int readout_request, bool rope = false) {
  Plan p{};
  p.kv_tile = in_dt == LA_BF16 ? 64 : 16;
  p.T = T < N ? T : N;
  p.nblk = N == 0 ? 0 : (N + p.T - 1) / p.T;
  p.sweep = in_dt == LA_BF16 && d < LA_READOUT_ITEMS_MIN_D && !rope;
  p.items = in_dt == LA_BF16 && (d >= LA_READOUT_ITEMS_MIN_D || rope);
  if (N == 0) return p;
  const long long bhc = static_cast<long long>(B) * H;
  const long long pairs = bhc * p.nblk;  // (b, h, block) pairs
  const int Tb = p.T;                    // tokens in a full block

  // KV splits per block
  const int ntiles = (Tb + p.kv_tile - 1) / p.kv_tile;
  long long s;
  if (request > 0) {
    s = request;
  } else {
    const long long target = d == 128 ? kKvTargetWorkgroups / 2
                             : rope    ? kKvRopeTargetWorkgroups
                                       : kKvTargetWorkgroups;
    s = (target + pairs - 1) / pairs;
    // of s - 1, s, s + 1 take the count whose grid ends closest to a whole
    // round of the CUs (ties: s); a grid of 2.25 workgroups per CU leaves
    // most of its last round idle
    const auto idle = [&](long long c) {
      const long long wg = pairs * c;
      return (kCUs - wg % kCUs) % kCUs;
    };
    long long best = s;
    for (long long c = s - 1; c <= s + 1; ++c)
      if (c >= 1 && idle(c) < idle(best)) best = c;
    s = best;
    const long long by_size = Tb / (kKvMinTokensPerFeature * (d + 1));
    s = s < by_size ? s : by_size;
  }
  if (s > ntiles) s = ntiles;
  // more than one split needs the partials in `out`: splits * (d*d + d) * 4
  // bytes per (b, h, block)
  const long long cap = static_cast<long long>(N) * d * elem_size(out_dt) /
                        (static_cast<long long>(p.nblk) * (d * d + d) * 4);
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  const int per = static_cast<int>((Tb + s - 1) / s);
  p.tps = (per + p.kv_tile - 1) / p.kv_tile * p.kv_tile;
  p.splits = (Tb + p.tps - 1) / p.tps;
  p.direct = p.nblk == 1 && p.splits == 1;
  p.in_place = p.nblk > 1 && p.splits == 1;
  // One block at d = 128 over enough heads to give every CU a workgroup:
  // quadrants of the state instead of token splits (no partials, no reduce).
  // A split request keeps the split path.
  if (in_dt == LA_BF16 && d == 128 && p.nblk == 1 && !rope && request <= 0 &&
      la::kv_quad_workgroups(bhc) >= kCUs && bhc >= kKvQuadMinPairs) {
    p.quad = true;
    p.splits = 1;
    p.tps = ((Tb + p.kv_tile - 1) / p.kv_tile) * p.kv_tile;
    p.direct = true;
  }

  // readout
  if (p.items) {
    const long long cap = static_cast<long long>(kCUs) *
                          (d == 128 ? la::readout_items_min_waves<128>()
                           : d == 64 ? la::readout_items_min_waves<64>()
                                     : la::readout_items_min_waves<32>());
    long long s2 = readout_request > 0 ? (readout_request + pairs - 1) / pairs
                                       : items_per_block(pairs, cap);
    // an item builds the state's operands (64 KB at d = 128) before it
    // streams: keep items at least kReadoutItemMinTokens long
    const long long by_len = Tb / kReadoutItemMinTokens;
    if (readout_request <= 0 && s2 > by_len) s2 = by_len;
    const long long tiles = (Tb + 63) / 64;
    if (s2 > tiles) s2 = tiles;
    if (s2 < 1) s2 = 1;
    p.ro_splits = static_cast<int>(s2);
    p.readout_wgs = static_cast<int>(pairs * s2 < cap ? pairs * s2 : cap);
  } else if (p.sweep) {
    const int unit = 4 * 16 * LA_READOUT_ROWS;
    p.units_per_block = (Tb + unit - 1) / unit;
    long long wgs = readout_request > 0 ? readout_request : kSweepWorkgroups;
    // Workgroup steps take runs of one unit when a block has at least as many
    // units as the grid has workgroups, else runs of two (which halve the
    // operand rebuilds).  Measured, one box: the 720p chunk 261.0 us with
    // single units against 263.4-264.8 with runs of two; the 480p chunk
    // stream 789-791 us per 12 calls with runs of two against 803 with single
    // units, the 480p global call 60.0 against 61.5, the 480p stream in one
    // call 685-692 against 695 us.
    p.run_log2 = p.units_per_block >= wgs ? 0 : 1;
    const int run = 1 << p.run_log2;
    const long long runs = (pairs * p.units_per_block + run - 1) / run;
    if (wgs > runs) wgs = runs;
    if (wgs < 1) wgs = 1;
    p.readout_wgs = static_cast<int>(wgs);
  } else {
    const int ro_unit = 128;  // readout_f32 processes 32-token tiles
    const long long target = readout_request > 0 ? readout_request
                             : d == 128            ? kReadoutTargetWorkgroups / 2
                                                   : kReadoutTargetWorkgroups;
    const long long per_block = (target + pairs - 1) / pairs;
    long long tpw = (Tb + per_block - 1) / per_block;
    if (tpw < 1) tpw = 1;
    tpw = (tpw + ro_unit - 1) / ro_unit * ro_unit;
    p.readout_tpw = static_cast<int>(tpw);
    p.readout_wgs = static_cast<int>(((Tb + tpw - 1) / tpw) * pairs);
  }
  return p;
}

int record(const la_launch_opts* o, int i, hipStream_t stream) {
  if (o == nullptr || o->stage_events == nullptr) return LA_OK;
  return hipEventRecord(o->stage_events[i], stream) == hipSuccess ? LA_OK : LA_E_HIP;
}

int launched() { return hipGetLastError() == hipSuccess ? LA_OK : LA_E_HIP; }

template <typename Kern>
int allow_smem(Kern* kern, size_t smem) {
  if (smem <= 65536) return LA_OK;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(smem)) == hipSuccess
             ? LA_OK
             : LA_E_HIP;
}

template <int D>
int launch_kv(const Plan& p, const void* k, const void* v, int in_dt, int B, int H, int N,
              const float* state_in, float* dst, const la::RopeGrid* rope, hipStream_t stream) {
  const dim3 grid(p.nblk * p.splits, H, B);
  if (rope != nullptr) {
    if (in_dt == LA_BF16)
      la::kv_partial_rope_bf16<D><<<grid, la::kv_threads<D>(), 0, stream>>>(
          static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), N, p.T, p.splits,
          p.tps, state_in, dst, *rope);
    else
      la::kv_partial_rope_f32<D><<<grid, la::kBlock, 0, stream>>>(
          static_cast<const float*>(k), static_cast<const float*>(v), N, p.T, p.splits, p.tps,
          state_in, dst, *rope);
    return launched();
  }
  if (p.quad) {
    if constexpr (D == 128) {
      const long long wgs = la::kv_quad_workgroups(static_cast<long long>(B) * H);
      la::kv_quad_bf16<<<static_cast<unsigned>(wgs), la::KvQuad::NT, 0, stream>>>(
          static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), N, B * H, state_in,
          dst);
      return launched();
    }
    return LA_E_UNSUPPORTED;
  }
  if (in_dt == LA_BF16)
    la::kv_partial_bf16<D><<<grid, la::kv_threads<D>(), 0, stream>>>(
        static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), N, p.T, p.splits, p.tps,
        state_in, dst);
  else
    la::kv_partial_f32<D><<<grid, la::kBlock, 0, stream>>>(
        static_cast<const float*>(k), static_cast<const float*>(v), N, p.T, p.splits, p.tps,
        state_in, dst);
  return launched();
}

template <int D>
int launch_readout_rope(const Plan& p, const void* q, int out_dt, int B, int H, int N,
                        const float* states, void* out, float eps, const la::RopeGrid& rope,
                        hipStream_t stream) {
  if (p.items) {
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const int items = B * H * p.nblk * p.ro_splits;
    if (out_dt == LA_BF16)
      la::readout_rope_bf16<D, true><<<p.readout_wgs, la::RowTile<D>::NT, 0, stream>>>(
          qq, states, out, N, p.T, p.nblk, p.ro_splits, items, eps, rope);
    else
      la::readout_rope_bf16<D, false><<<p.readout_wgs, la::RowTile<D>::NT, 0, stream>>>(
          qq, states, out, N, p.T, p.nblk, p.ro_splits, items, eps, rope);
    return launched();
  }
  const dim3 grid(p.nblk * ((p.T + p.readout_tpw - 1) / p.readout_tpw), H, B);
  const float* qq = static_cast<const float*>(q);
  constexpr size_t smem = la::readout_rope_f32_smem<D>();
  int rc;
  if (out_dt == LA_BF16) {
    if ((rc = allow_smem(&la::readout_rope_f32<D, true>, smem)) != LA_OK) return rc;
    la::readout_rope_f32<D, true><<<grid, la::kBlock, smem, stream>>>(
        qq, states, out, N, p.T, p.nblk, p.readout_tpw, eps, rope);
  } else {
    if ((rc = allow_smem(&la::readout_rope_f32<D, false>, smem)) != LA_OK) return rc;
    la::readout_rope_f32<D, false><<<grid, la::kBlock, smem, stream>>>(
        qq, states, out, N, p.T, p.nblk, p.readout_tpw, eps, rope);
  }
  return launched();
}

template <int D>
int launch_readout(const Plan& p, const void* q, int out_dt, int B, int H, int N,
                   const float* states, void* out, float eps, const la::RopeGrid* rope,
                   hipStream_t stream) {
  if (rope != nullptr)
    return launch_readout_rope<D>(p, q, out_dt, B, H, N, states, out, eps, *rope, stream);
  if (p.items) {
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const int items = B * H * p.nblk * p.ro_splits;
    if (out_dt == LA_BF16)
      la::readout_items_bf16<D, true><<<p.readout_wgs, la::RowTile<D>::NT, 0, stream>>>(
          qq, states, out, N, p.T, p.nblk, p.ro_splits, items, eps);
    else
      la::readout_items_bf16<D, false><<<p.readout_wgs, la::RowTile<D>::NT, 0, stream>>>(
          qq, states, out, N, p.T, p.nblk, p.ro_splits, items, eps);
    return launched();
  }
  if (p.sweep) {
    // only d below LA_READOUT_ITEMS_MIN_D plans the sweep: nothing else is built
    if constexpr (D < LA_READOUT_ITEMS_MIN_D) {
      const uint16_t* qq = static_cast<const uint16_t*>(q);
      const int total = B * H * p.nblk * p.units_per_block;
      constexpr int nt = la::sweep_threads<D>();
      if (out_dt == LA_BF16)
        la::readout_sweep_bf16<D, true><<<p.readout_wgs, nt, 0, stream>>>(
            qq, states, out, N, p.T, p.nblk, p.units_per_block, total, p.run_log2, eps);
      else
        la::readout_sweep_bf16<D, false><<<p.readout_wgs, nt, 0, stream>>>(
            qq, states, out, N, p.T, p.nblk, p.units_per_block, total, p.run_log2, eps);
      return launched();
    }
    return LA_E_UNSUPPORTED;
  }
  // float32 queries: workgroups over contiguous token ranges of one block
  const dim3 grid(p.nblk * ((p.T + p.readout_tpw - 1) / p.readout_tpw), H, B);
  const float* qq = static_cast<const float*>(q);
  constexpr size_t smem = la::readout_f32_smem<D>();
  if (out_dt == LA_BF16) {
    if (smem > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&la::readout_f32<D, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, smem) != hipSuccess)
      return LA_E_HIP;
    la::readout_f32<D, true><<<grid, la::kBlock, smem, stream>>>(qq, states, out, N, p.T, p.nblk,
                                                                 p.readout_tpw, eps);
  } else {
    if (smem > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&la::readout_f32<D, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, smem) != hipSuccess)
      return LA_E_HIP;
    la::readout_f32<D, false><<<grid, la::kBlock, smem, stream>>>(qq, states, out, N, p.T, p.nblk,
                                                                  p.readout_tpw, eps);
  }
  return launched();
}

// The three stages for any number of blocks.  `states` holds nblk states per
// (b, h) (one for the chunk and global calls).
template <int D>
int run(const Plan& p, const void* q, const void* k, const void* v, const float* state_in,
        void* out, float* states, int B, int H, int N, int in_dt, int out_dt, float eps,
        const la::RopeGrid* rope, const la_launch_opts* opts, hipStream_t stream) {
  constexpr int E = D * D + D;
  const int n4 = E / 4;
  int rc;
  if ((rc = record(opts, 0, stream)) != LA_OK) return rc;
  float* partials = p.direct || p.in_place ? states : static_cast<float*>(out);
  if (p.nblk >= 1) {
    if ((rc = launch_kv<D>(p, k, v, in_dt, B, H, N, state_in, partials, rope, stream)) != LA_OK)
      return rc;
  }
  if ((rc = record(opts, 1, stream)) != LA_OK) return rc;
  if (p.nblk <= 1 && !p.direct) {
    // one block (or an empty chunk): partial sums plus S_in
    const dim3 grid((n4 + la::kWave - 1) / la::kWave, H, B);
    la::state_reduce<<<grid, la::kBlock, 0, stream>>>(
        reinterpret_cast<const float4*>(partials), p.nblk == 1 ? p.splits : 0, n4,
        reinterpret_cast<const float4*>(state_in), reinterpret_cast<float4*>(states));
    if ((rc = launched()) != LA_OK) return rc;
  } else if (p.nblk > 1) {
    const dim3 grid((n4 + la::kBlock - 1) / la::kBlock, H, B);
    la::state_scan<<<grid, la::kBlock, 0, stream>>>(
        reinterpret_cast<const float4*>(partials), p.nblk, p.splits, n4,
        reinterpret_cast<const float4*>(state_in), reinterpret_cast<float4*>(states));
    if ((rc = launched()) != LA_OK) return rc;
  }
  if ((rc = record(opts, 2, stream)) != LA_OK) return rc;
  if (N > 0) {
    if ((rc = launch_readout<D>(p, q, out_dt, B, H, N, states, out, eps, rope, stream)) != LA_OK)
      return rc;
  }
  return record(opts, 3, stream);
}

// ---------------------------------------------------------------------------
// Backward.  Workspace layout: R [B][H][blocks][d*d + d] float32 (the suffix
// sums), then, when the query kernel uses more than one split per block,
// its partials [B][H][blocks][splits][d*d + d].
struct BwdPlan {
  int nblk;        // blocks (0 when N == 0)
  int T;           // tokens per block
  int qs;          // query-gradient items (splits) per block
  int qgrid;       // its grid (bf16: persistent, <= items)
  int qtps;        // float32: tokens per split
  int ks;          // key-gradient items per block
  int kgrid;       // its grid (bf16: persistent)
  int ktps;
  bool ksweep;     // bwd_key_sweep_bf16 instead of the work items
  int kupb;        // its units per block
  size_t ws_bytes; // workspace the plan needs
};

// Whether the planner gives a backward call the key-gradient sweep (bf16
// inputs at d <= 64 without rotary and without a key-workgroup request).
bool bwd_key_sweep(int d, int in_dt, bool rope) {
  return LA_BWDK_SWEEP && in_dt == LA_BF16 && d <= 64 && !rope;
}

// ws_avail: the caller's workspace size (SIZE_MAX when planning the size).
// rope: the rotary kernels (the key kernel's grid differs; the workspace,
// set by the query splits alone, does not).
BwdPlan make_bwd_plan(int B, int H, int N, int T, int d, int in_dt, int qrequest, int krequest,
                      size_t ws_avail, bool rope = false) {
  BwdPlan p{};
  p.T = T < N ? T : N;
  p.nblk = N == 0 ? 0 : (N + p.T - 1) / p.T;
  if (N == 0) return p;
  const bool bf = in_dt == LA_BF16;
  const int tile = bf ? 64 : 16;
  const long long pairs = static_cast<long long>(B) * H * p.nblk;
  const size_t st = static_cast<size_t>(d) * d + d;
  const size_t r_bytes = static_cast<size_t>(pairs) * st * sizeof(float);
  const int Tb = p.T;
  const int ntiles = (Tb + tile - 1) / tile;

  // query-gradient splits (each writes one partial state gradient)
  long long s;
  if (qrequest > 0) {
    s = qrequest;
  } else if (bf) {
    s = items_per_block(pairs, bwd_query_capacity(d));
  } else {
    s = (kBwdF32TargetWorkgroups + pairs - 1) / pairs;
  }
  const long long by_size = Tb / (kKvMinTokensPerFeature * (d + 1));
  if (qrequest <= 0 && s > by_size) s = by_size;
  if (s > ntiles) s = ntiles;
  if (s > 1 && ws_avail != SIZE_MAX) {
    // splits + 1 state-sized slots per (b, h, block)
    const size_t slots = ws_avail / r_bytes;
    const long long most = slots > 1 ? static_cast<long long>(slots - 1) : 1;
    if (s > most) s = most;
  }
  if (s < 1) s = 1;
  if (bf) {
    p.qs = static_cast<int>(s);
    const long long items = pairs * s;
    p.qgrid = static_cast<int>(items < bwd_query_capacity(d) ? items : bwd_query_capacity(d));
  } else {
    const int per = static_cast<int>((Tb + s - 1) / s);
    p.qtps = (per + tile - 1) / tile * tile;
    p.qs = (Tb + p.qtps - 1) / p.qtps;
  }
  p.ws_bytes = p.qs > 1 ? r_bytes * (p.qs + 1) : r_bytes;

  // key-gradient items
  long long kw;
  if (krequest > 0) {
    kw = (krequest + pairs - 1) / pairs;
  } else if (bf) {
    kw = items_per_block(pairs, bwd_key_capacity(d, rope));
  } else {
    kw = (kBwdF32TargetWorkgroups + pairs - 1) / pairs;
  }
  if (kw > ntiles) kw = ntiles;
  if (kw < 1) kw = 1;
  if (bf) {
    p.ks = static_cast<int>(kw);
    const long long items = pairs * kw;
    const int cap = bwd_key_capacity(d, rope);
    p.kgrid = static_cast<int>(items < cap ? items : cap);
  } else {
    const int per = static_cast<int>((Tb + kw - 1) / kw);
    p.ktps = (per + tile - 1) / tile * tile;
    p.ks = (Tb + p.ktps - 1) / p.ktps;
  }
  // bf16 at d <= 64 without a key-item request: the sweep
  if (bwd_key_sweep(d, in_dt, rope) && krequest <= 0) {
    const int unit = la::KeySweep<64>::UNIT;
    p.ksweep = true;
    p.kupb = (Tb + unit - 1) / unit;
    const long long units = pairs * p.kupb;
    p.kgrid = static_cast<int>(units < kBwdKeySweepWorkgroups ? units : kBwdKeySweepWorkgroups);
  }
  return p;
}

template <int D, bool GO_BF16>
int launch_bwd_query(const BwdPlan& p, const void* q, const void* dout, const float* states,
                     void* dq, int in_dt, int B, int H, int N, float eps, float* dst,
                     const la::RopeGrid* rope, hipStream_t stream) {
  if (rope != nullptr) {
    if (in_dt == LA_BF16) {
      const int items = B * H * p.nblk * p.qs;
      la::bwd_query_rope_bf16<D, GO_BF16><<<p.qgrid, la::RowTile<D>::NT, 0, stream>>>(
          static_cast<const uint16_t*>(q), dout, states, dq, N, p.T, p.nblk, p.qs, items, eps,
          dst, *rope);
    } else {
      const dim3 grid(p.nblk * p.qs, H, B);
      constexpr size_t smem = la::bwd_query_rope_f32_smem<D>();
      const int rc = allow_smem(&la::bwd_query_rope_f32<D, GO_BF16>, smem);
      if (rc != LA_OK) return rc;
      la::bwd_query_rope_f32<D, GO_BF16><<<grid, la::kBlock, smem, stream>>>(
          static_cast<const float*>(q), dout, states, dq, N, p.T, p.qs, p.qtps, eps, dst, *rope);
    }
    return launched();
  }
  if (in_dt == LA_BF16) {
    const int items = B * H * p.nblk * p.qs;
    la::bwd_query_bf16<D, GO_BF16><<<p.qgrid, la::RowTile<D>::NT, 0, stream>>>(
        static_cast<const uint16_t*>(q), dout, states, dq, N, p.T, p.nblk, p.qs, items, eps, dst);
  } else {
    const dim3 grid(p.nblk * p.qs, H, B);
    constexpr size_t smem = la::bwd_query_f32_smem<D>();
    const int rc = allow_smem(&la::bwd_query_f32<D, GO_BF16>, smem);
    if (rc != LA_OK) return rc;
    la::bwd_query_f32<D, GO_BF16><<<grid, la::kBlock, smem, stream>>>(
        static_cast<const float*>(q), dout, states, dq, N, p.T, p.qs, p.qtps, eps, dst);
  }
  return launched();
}

template <int D, bool GO_BF16>
int launch_bwd_key(const BwdPlan& p, const void* k, const void* v, const float* R, void* dk,
                   void* dv, int in_dt, int B, int H, int N, const la::RopeGrid* rope,
                   hipStream_t stream) {
  if (rope != nullptr) {
    if (in_dt == LA_BF16) {
      const int items = B * H * p.nblk * p.ks;
      la::bwd_key_rope_bf16<D, GO_BF16><<<p.kgrid, la::RowTile<D>::NT, 0, stream>>>(
          static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), R, dk, dv, N, p.T,
          p.nblk, p.ks, items, *rope);
    } else {
      const dim3 grid(p.nblk * p.ks, H, B);
      constexpr size_t smem = la::bwd_key_rope_f32_smem<D>();
      const int rc = allow_smem(&la::bwd_key_rope_f32<D, GO_BF16>, smem);
      if (rc != LA_OK) return rc;
      la::bwd_key_rope_f32<D, GO_BF16><<<grid, la::kBlock, smem, stream>>>(
          static_cast<const float*>(k), static_cast<const float*>(v), R, dk, dv, N, p.T, p.ks,
          p.ktps, *rope);
    }
    return launched();
  }
  if constexpr (D <= 64) {
    if (p.ksweep) {
      const int total = B * H * p.nblk * p.kupb;
      la::bwd_key_sweep_bf16<D, GO_BF16><<<p.kgrid, la::RowTile<D>::NT, 0, stream>>>(
          static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), R, dk, dv, N, p.T,
          p.nblk, p.kupb, total);
      return launched();
    }
  }
  if (in_dt == LA_BF16) {
    const int items = B * H * p.nblk * p.ks;
    la::bwd_key_bf16<D, GO_BF16><<<p.kgrid, la::RowTile<D>::NT, 0, stream>>>(
        static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), R, dk, dv, N, p.T,
        p.nblk, p.ks, items);
  } else {
    const dim3 grid(p.nblk * p.ks, H, B);
    constexpr size_t smem = la::bwd_key_f32_smem<D>();
    const int rc = allow_smem(&la::bwd_key_f32<D, GO_BF16>, smem);
    if (rc != LA_OK) return rc;
    la::bwd_key_f32<D, GO_BF16><<<grid, la::kBlock, smem, stream>>>(
        static_cast<const float*>(k), static_cast<const float*>(v), R, dk, dv, N, p.T, p.ks,
        p.ktps);
  }
  return launched();
}

template <int D, bool GO_BF16>
int run_bwd(const BwdPlan& p, const void* q, const void* k, const void* v, const float* states,
            const void* dout, const float* dstates, void* dq, void* dk, void* dv,
            float* dstate_in, int B, int H, int N, int in_dt, float eps, void* workspace,
            const la::RopeGrid* rope, const la_launch_opts* opts, hipStream_t stream) {
  constexpr int E = D * D + D;
  const int n4 = E / 4;
  float* R = static_cast<float*>(workspace);
  float* partials = p.qs > 1 ? R + static_cast<size_t>(B) * H * p.nblk * E : R;
  int rc;
  if ((rc = record(opts, 0, stream)) != LA_OK) return rc;
  if ((rc = launch_bwd_query<D, GO_BF16>(p, q, dout, states, dq, in_dt, B, H, N, eps, partials,
                                         rope, stream)) != LA_OK)
    return rc;
  if ((rc = record(opts, 1, stream)) != LA_OK) return rc;
  const dim3 grid((n4 + la::kBlock - 1) / la::kBlock, H, B);
  la::state_suffix_scan<<<grid, la::kBlock, 0, stream>>>(
      reinterpret_cast<const float4*>(partials), p.nblk, p.qs, n4,
      reinterpret_cast<const float4*>(dstates), reinterpret_cast<float4*>(R),
      reinterpret_cast<float4*>(dstate_in));
  if ((rc = launched()) != LA_OK) return rc;
  if ((rc = record(opts, 2, stream)) != LA_OK) return rc;
  if ((rc = launch_bwd_key<D, GO_BF16>(p, k, v, R, dk, dv, in_dt, B, H, N, rope, stream)) !=
      LA_OK)
    return rc;
  return record(opts, 3, stream);
}

// Checks of a rotary call's grid (none for a plain call): token indices (plus
// a tile of padding) below 2^22, where the kernels' float divisions are
// exact, and every frame index exact in float.
int check_rope(const la::RopeGrid* rope, int N) {
  if (rope == nullptr) return LA_OK;
  if (rope->gh <= 0 || rope->gw <= 0 ||
      static_cast<long long>(rope->gh) * rope->gw >= kRopeMaxTokens)
    return LA_E_INVAL;
  if (N >= kRopeMaxTokens - 64 || rope->frame0 <= -kRopeMaxTokens ||
      rope->frame0 >= kRopeMaxTokens)
    return LA_E_INVAL;
  if (!(rope->theta > 0.0f) || !isfinite(rope->theta)) return LA_E_INVAL;
  return LA_OK;
}

// Whether a backward call of this shape runs its two halves of (b, h) pairs on
// two streams (outside stream capture, without stage events, with the
// device's second stream available; see backward()).  Only calls whose
// key-gradient kernel works on items: the sweep takes the whole GPU by itself
// (the 720p chunk: 666 us per call on one stream, 686 us with two).
bool bwd_two_streams(int B, int H, int N, int d, int in_dt, bool rope) {
  const long long P = static_cast<long long>(B) * H;
  return in_dt == LA_BF16 && !bwd_key_sweep(d, in_dt, rope) && P >= 2 && P - P / 2 <= 65535 &&
         N > 0 && P * static_cast<long long>(N) >= kBwdSplitMinTokens;
}

// run_bwd for the head dimension and gradient type of a call.
int run_bwd_d(int d, bool gb, const BwdPlan& p, const void* q, const void* k, const void* v,
              const float* states, const void* dout, const float* dstates, void* dq, void* dk,
              void* dv, float* dstate_in, int B, int H, int N, int in_dt, float eps,
              void* workspace, const la::RopeGrid* rope, const la_launch_opts* opts,
              hipStream_t stream) {
#define LA_RUN_BWD(DD)                                                                          \
  return gb ? run_bwd<DD, true>(p, q, k, v, states, dout, dstates, dq, dk, dv, dstate_in, B, H, \
                                N, in_dt, eps, workspace, rope, opts, stream)                   \
            : run_bwd<DD, false>(p, q, k, v, states, dout, dstates, dq, dk, dv, dstate_in, B, H,\
                                 N, in_dt, eps, workspace, rope, opts, stream)
  switch (d) {
    case 32:
      LA_RUN_BWD(32);
    case 64:
      LA_RUN_BWD(64);
    default:
      LA_RUN_BWD(128);
  }
#undef LA_RUN_BWD
}

// Checks shared by every backward call, then the launches.  The sequence of
// N tokens per (b, h) is cut into blocks of T (one block: T >= N); `states`
// holds the forward's state after every block.  `empty_block`: the chunk
// call with L = 0 (one block of no tokens, so dstate_in = dstates).
int backward(const void* q, const void* k, const void* v, const float* states, const void* dout,
             const float* dstates, void* dq, void* dk, void* dv, float* dstate_in, int B, int H,
             int N, int T, int d, int in_dt, int grad_dt, float eps, void* workspace,
             size_t workspace_bytes, bool empty_block, const la_launch_opts* opts,
             hipStream_t stream, const la::RopeGrid* rope = nullptr,
             bool static_scratch = false) {
  int rc = check_shape(B, H, N, d, in_dt, grad_dt);
  if (rc != LA_OK) return rc;
  if (T <= 0) return LA_E_INVAL;
  if ((rc = check_sizes(B, H, N, T, d)) != LA_OK) return rc;
  if ((rc = check_rope(rope, N)) != LA_OK) return rc;
  if (!(eps >= 0.0f) || !isfinite(eps)) return LA_E_INVAL;
  if (N > 0 && (q == nullptr || k == nullptr || v == nullptr || states == nullptr ||
                dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr))
    return LA_E_INVAL;
  if (empty_block && states == nullptr) return LA_E_INVAL;
  const void* ptrs[] = {q, k, v, states, dout, dstates, dq, dk, dv, dstate_in, workspace};
  for (const void* ptr : ptrs)
    if (ptr != nullptr && !aligned16(ptr)) return LA_E_ALIGN;

  const int nblk = N == 0 ? (empty_block ? 1 : 0) : (N + (T < N ? T : N) - 1) / (T < N ? T : N);
  const size_t bh = static_cast<size_t>(B) * H;
  const size_t st = (static_cast<size_t>(d) * d + d) * sizeof(float);
  // static_scratch: the workspace is this device's `scratch` (the caller
  // passes none); the plan fits its split count to that array
  if (static_scratch) {
    if (workspace != nullptr || workspace_bytes != 0) return LA_E_INVAL;
    workspace_bytes = LA_NOALLOC_SCRATCH_BYTES;
  }
  const size_t in_bytes = bh * N * d * elem_size(in_dt);
  const size_t g_bytes = bh * N * d * elem_size(grad_dt);
  BwdPlan p = empty_block
                  ? make_bwd_plan(B, H, 1, 1, d, in_dt, 1, 1, SIZE_MAX)
                  : make_bwd_plan(B, H, N, T, d, in_dt, opts ? opts->kv_splits : 0,
                                  opts ? opts->readout_workgroups : 0, workspace_bytes,
                                  rope != nullptr);
  if (empty_block) {
    p.T = 1;  // one block of no tokens: every workgroup's range is empty
  }
  const size_t need = nblk == 0 ? 0 : p.ws_bytes;
  if (static_scratch) {
    if (need > LA_NOALLOC_SCRATCH_BYTES) return LA_E_SCRATCH;
  } else if (need > 0 && (workspace == nullptr || workspace_bytes < need)) {
    return LA_E_INVAL;
  }

  // outputs against inputs and against each other
  struct Buf {
    const void* p;
    size_t n;
  };
  const Buf ins[] = {{q, in_bytes}, {k, in_bytes}, {v, in_bytes}, {states, st * bh * nblk},
                     {dout, g_bytes}, {dstates, st * bh * nblk}};
  const Buf outs[] = {{dq, g_bytes}, {dk, g_bytes}, {dv, g_bytes}, {dstate_in, st * bh},
                      {workspace, need}};
  for (const Buf& o : outs) {
    for (const Buf& i : ins)
      if (overlaps(o.p, o.n, i.p, i.n)) return LA_E_ALIAS;
    for (const Buf& o2 : outs)
      if (&o2 != &o && overlaps(o.p, o.n, o2.p, o2.n)) return LA_E_ALIAS;
  }

  if (nblk == 0) {
    if (dstate_in != nullptr) {
      const size_t n4 = bh * (static_cast<size_t>(d) * d + d) / 4;
      size_t blocks = (n4 + la::kBlock - 1) / la::kBlock;
      if (blocks > 4096) blocks = 4096;
      la::fill_zero<<<static_cast<unsigned>(blocks), la::kBlock, 0, stream>>>(
          reinterpret_cast<float4*>(dstate_in), n4);
      return launched();
    }
    return LA_OK;
  }
  if (static_scratch && (rc = device_scratch(stream, &workspace)) != LA_OK) return rc;
  const bool gb = grad_dt == LA_BF16;

  // Two halves of the (b, h) pairs, each with its own plan, on two streams at
  // once: the caller's stream and this device's second stream (AuxStream).
  // On one stream the query-gradient kernel (bound by its own latency and VALU
  // work) and the key-gradient kernel (bound by its writes) run one after the
  // other, and each kernel's last round of workgroups leaves compute units
  // idle; with two, each half's kernels fill the compute units the other's
  // leave idle, and one half's key kernel can run beside the other's query
  // kernel.  Measured per call with the work-item key kernel: the 720p chunk
  // 690 us against 699-701 us on one stream, the rotary backward 706-707
  // against 721-724 us, the 480p stream in one call 1,762 against 1,767 us.
  // (Forking the second half only after the first half's query kernel:
  // 783 us.)  Calls that take the key-gradient sweep stay on one stream
  // (bwd_two_streams).  Each half keeps the whole
  // call's query splits per (b, h), so every result is bitwise that of one
  // stream, and the halves' workspaces tile exactly the one the whole call
  // needs.  Not taken for the float32 path, for the static scratch, for small
  // calls, under stream capture (one stream is captured as it is), or when
  // stage events are asked for (they time the kernels of one stream).
  const long long P = static_cast<long long>(bh);
  if (!static_scratch && !empty_block && bwd_two_streams(B, H, N, d, in_dt, rope != nullptr) &&
      (opts == nullptr || opts->stage_events == nullptr)) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    AuxStream* aux = nullptr;
    if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone)
      aux = aux_stream(stream);
    const int pa = static_cast<int>(P / 2), pb = static_cast<int>(P - P / 2);
    const int kreq = opts ? opts->readout_workgroups : 0;
    const BwdPlan plan_a = make_bwd_plan(1, pa, N, T, d, in_dt, p.qs, kreq, SIZE_MAX,
                                         rope != nullptr);
    const BwdPlan plan_b = make_bwd_plan(1, pb, N, T, d, in_dt, p.qs, kreq, SIZE_MAX,
                                         rope != nullptr);
    if (aux != nullptr && plan_a.qs == p.qs && plan_b.qs == p.qs &&
        plan_a.ws_bytes + plan_b.ws_bytes <= need) {
      // half B starts pa pairs in: its tokens, states and workspace follow half A's
      const size_t tok = static_cast<size_t>(pa) * N * d;
      const size_t sts = static_cast<size_t>(pa) * nblk * (static_cast<size_t>(d) * d + d);
      const size_t st1 = static_cast<size_t>(pa) * (static_cast<size_t>(d) * d + d);
      const size_t ie = elem_size(in_dt), ge = elem_size(grad_dt);
      auto at = [](const void* x, size_t bytes) -> void* {
        return x == nullptr ? nullptr
                            : static_cast<char*>(const_cast<void*>(x)) + bytes;
      };
      auto atf = [](const float* x, size_t n) -> float* {
        return x == nullptr ? nullptr : const_cast<float*>(x) + n;
      };
      std::lock_guard<std::mutex> lock(aux->mu);
      if (hipEventRecord(aux->fork, stream) != hipSuccess ||
          hipStreamWaitEvent(aux->s, aux->fork, 0) != hipSuccess)
        return LA_E_HIP;
      const int rc_a = run_bwd_d(d, gb, plan_a, q, k, v, states, dout, dstates, dq, dk, dv,
                                 dstate_in, 1, pa, N, in_dt, eps, workspace, rope, opts, stream);
      const int rc_b =
          rc_a != LA_OK
              ? rc_a
              : run_bwd_d(d, gb, plan_b, at(q, tok * ie), at(k, tok * ie), at(v, tok * ie),
                          atf(states, sts), at(dout, tok * ge), atf(dstates, sts),
                          at(dq, tok * ge), at(dk, tok * ge), at(dv, tok * ge),
                          atf(dstate_in, st1), 1, pb, N, in_dt, eps,
                          at(workspace, plan_a.ws_bytes), rope, opts, aux->s);
      // join even after an error: the caller's stream never runs ahead of
      // work already on the second stream
      const bool joined = hipEventRecord(aux->join, aux->s) == hipSuccess &&
                          hipStreamWaitEvent(stream, aux->join, 0) == hipSuccess;
      if (rc_a != LA_OK) return rc_a;
      if (rc_b != LA_OK) return rc_b;
      return joined ? LA_OK : LA_E_HIP;
    }
  }
  return run_bwd_d(d, gb, p, q, k, v, states, dout, dstates, dq, dk, dv, dstate_in, B, H, N,
                   in_dt, eps, workspace, rope, opts, stream);
}

// ---------------------------------------------------------------------------
// Temporal convolution: checks, then one launch.  one_chunk: the chunk call
// (cache_out may be cache_in).
int temporal_conv(const void* x, const void* cache_in, const float* w, const float* bias, void* y,
                  void* cache_out, int B, int F, int Tf, int P, int C, int x_dt, int y_dt,
                  hipStream_t stream) {
  if (B <= 0 || F < 0 || P <= 0 || C <= 0 || Tf <= 0) return LA_E_INVAL;
  if (C % 8 != 0) return LA_E_UNSUPPORTED;
  using ull = unsigned long long;
  if (!bytes_below_limit({static_cast<ull>(B), static_cast<ull>(F), static_cast<ull>(P),
                          static_cast<ull>(C), 4}) ||
      !bytes_below_limit({static_cast<ull>(B), static_cast<ull>(P), static_cast<ull>(C), 4}))
    return LA_E_INVAL;
  if ((x_dt != LA_F32 && x_dt != LA_BF16) || (y_dt != LA_F32 && y_dt != LA_BF16))
    return LA_E_UNSUPPORTED;
  if (w == nullptr || (F > 0 && (x == nullptr || y == nullptr))) return LA_E_INVAL;
  const long long nchunks = F == 0 ? 1 : (static_cast<long long>(F) + Tf - 1) / Tf;
  const long long cols = static_cast<long long>(B) * P * (C / 8);
  if (nchunks > 65535 || (cols + la::kBlock - 1) / la::kBlock > 0x7FFFFFFFLL) return LA_E_INVAL;
  const void* ptrs[] = {x, cache_in, w, bias, y, cache_out};
  for (const void* ptr : ptrs)
    if (ptr != nullptr && !aligned16(ptr)) return LA_E_ALIGN;
  const size_t xb = static_cast<size_t>(B) * F * P * C * elem_size(x_dt);
  const size_t yb = static_cast<size_t>(B) * F * P * C * elem_size(y_dt);
  const size_t cb = static_cast<size_t>(B) * P * C * elem_size(x_dt);
  const size_t wb = static_cast<size_t>(C) * 3 * sizeof(float);
  const size_t bb = static_cast<size_t>(C) * sizeof(float);
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, cache_in, cb) || overlaps(y, yb, cache_out, cb) ||
      overlaps(y, yb, w, wb) || overlaps(y, yb, bias, bb) || overlaps(cache_out, cb, x, xb) ||
      overlaps(cache_out, cb, w, wb) || overlaps(cache_out, cb, bias, bb))
    return LA_E_ALIAS;
  // the cache may be updated in place only when one thread reads and writes
  // each element (a single chunk)
  if (overlaps(cache_out, cb, cache_in, cb) && !(cache_out == cache_in && nchunks == 1))
    return LA_E_ALIAS;

  const dim3 grid(static_cast<unsigned>((cols + la::kBlock - 1) / la::kBlock),
                  static_cast<unsigned>(nchunks));
  const int C8 = C / 8;
  const bool xb16 = x_dt == LA_BF16, yb16 = y_dt == LA_BF16;
  if (xb16 && yb16)
    la::temporal_conv<true, true><<<grid, la::kBlock, 0, stream>>>(x, cache_in, w, bias, y, cache_out,
                                                                  F, Tf, P, C8, cols);
  else if (xb16)
    la::temporal_conv<true, false><<<grid, la::kBlock, 0, stream>>>(x, cache_in, w, bias, y,
                                                                   cache_out, F, Tf, P, C8, cols);
  else if (yb16)
    la::temporal_conv<false, true><<<grid, la::kBlock, 0, stream>>>(x, cache_in, w, bias, y,
                                                                   cache_out, F, Tf, P, C8, cols);
  else
    la::temporal_conv<false, false><<<grid, la::kBlock, 0, stream>>>(x, cache_in, w, bias, y,
                                                                    cache_out, F, Tf, P, C8, cols);
  return launched();
}

// Checks shared by every forward call, then the launches.  `need_state_in`:
// the chunk call requires it; the global and block-causal calls take NULL as
// zero.  `states_blocks`: number of states `states` holds per (b, h).
int forward(const void* q, const void* k, const void* v, const float* state_in,
            bool need_state_in, bool blockcausal, void* out, float* states, int B, int H, int N,
            int T, int d, int in_dt, int out_dt, float eps, const la_launch_opts* opts,
            hipStream_t stream, const la::RopeGrid* rope = nullptr) {
  int rc = check_shape(B, H, N, d, in_dt, out_dt);
  if (rc != LA_OK) return rc;
  if (T <= 0) return LA_E_INVAL;
  if ((rc = check_sizes(B, H, N, T, d)) != LA_OK) return rc;
  if ((rc = check_rope(rope, N)) != LA_OK) return rc;
  if (!(eps >= 0.0f) || !isfinite(eps)) return LA_E_INVAL;
  if (states == nullptr || (need_state_in && state_in == nullptr)) return LA_E_INVAL;
  if (N > 0 && (q == nullptr || k == nullptr || v == nullptr || out == nullptr)) return LA_E_INVAL;
  const void* ptrs[] = {q, k, v, out, state_in, states};
  for (const void* ptr : ptrs)
    if (ptr != nullptr && !aligned16(ptr)) return LA_E_ALIGN;

  const int nblk = N == 0 ? 1 : (N + (T < N ? T : N) - 1) / (T < N ? T : N);
  const size_t bh = static_cast<size_t>(B) * H;
  const size_t in_bytes = bh * N * d * elem_size(in_dt);
  const size_t out_bytes = bh * N * d * elem_size(out_dt);
  const size_t st_bytes = bh * (static_cast<size_t>(d) * d + d) * sizeof(float);
  const size_t sts_bytes = st_bytes * nblk;
  if (N > 0) {
    const void* ins[] = {q, k, v};
    for (const void* ptr : ins)
      if (overlaps(out, out_bytes, ptr, in_bytes) || overlaps(states, sts_bytes, ptr, in_bytes))
        return LA_E_ALIAS;
    if (overlaps(out, out_bytes, states, sts_bytes) ||
        overlaps(out, out_bytes, state_in, st_bytes))
      return LA_E_ALIAS;
  }
  // one block: state_in may be the state itself (in-place commit)
  if (nblk == 1 ? (state_in != states && overlaps(state_in, st_bytes, states, sts_bytes))
                : overlaps(state_in, st_bytes, states, sts_bytes))
    return LA_E_ALIAS;

  // a block-causal sequence of no tokens has no blocks and no states
  if (blockcausal && N == 0) return LA_OK;
  const Plan p = make_plan(B, H, N, T, d, in_dt, out_dt, opts ? opts->kv_splits : 0,
                           opts ? opts->readout_workgroups : 0, rope != nullptr);
  switch (d) {
    case 32:
      return run<32>(p, q, k, v, state_in, out, states, B, H, N, in_dt, out_dt, eps, rope, opts,
                     stream);
    case 64:
      return run<64>(p, q, k, v, state_in, out, states, B, H, N, in_dt, out_dt, eps, rope, opts,
                     stream);
    default:
      return run<128>(p, q, k, v, state_in, out, states, B, H, N, in_dt, out_dt, eps, rope, opts,
                      stream);
  }
}

la::RopeGrid rope_grid(int frame0, int grid_h, int grid_w, float theta) {
  la::RopeGrid g{};
  g.frame0 = frame0;
  g.gh = grid_h;
  g.gw = grid_w;
  g.hw = grid_h > 0 && grid_w > 0 && static_cast<long long>(grid_h) * grid_w < kRopeMaxTokens
             ? grid_h * grid_w
             : 0;
  g.rcp_hw = g.hw > 0 ? static_cast<float>(1.0 / g.hw) : 0.0f;
  g.rcp_gw = grid_w > 0 ? static_cast<float>(1.0 / grid_w) : 0.0f;
  g.theta = theta;
  return g;
}

}  // namespace

extern "C" {

int la_state_reset(float* state, int B, int H, int d, hipStream_t stream) {
  if (B <= 0 || H <= 0 || B > 65535 || H > 65535) return LA_E_INVAL;
  if (d != 32 && d != 64 && d != 128) return LA_E_UNSUPPORTED;
  if (state == nullptr) return LA_E_INVAL;
  if (!aligned16(state)) return LA_E_ALIGN;
  const size_t n4 = static_cast<size_t>(B) * H * (static_cast<size_t>(d) * d + d) / 4;
  size_t blocks = (n4 + la::kBlock - 1) / la::kBlock;
  if (blocks > 4096) blocks = 4096;
  la::fill_zero<<<static_cast<unsigned>(blocks), la::kBlock, 0, stream>>>(
      reinterpret_cast<float4*>(state), n4);
  return launched();
}

int la_chunk_forward(const void* q, const void* k, const void* v, const float* state_in, void* out,
                     float* state_out, int B, int H, int L, int d, int in_dt, int out_dt, float eps,
                     hipStream_t stream) {
  return forward(q, k, v, state_in, true, false, out, state_out, B, H, L, L > 0 ? L : 1, d, in_dt, out_dt,
                 eps, nullptr, stream);
}

int la_chunk_forward_ex(const void* q, const void* k, const void* v, const float* state_in,
                        void* out, float* state_out, int B, int H, int L, int d, int in_dt,
                        int out_dt, float eps, const la_launch_opts* opts, hipStream_t stream) {
  return forward(q, k, v, state_in, true, false, out, state_out, B, H, L, L > 0 ? L : 1, d, in_dt, out_dt,
                 eps, opts, stream);
}

int la_global_forward(const void* q, const void* k, const void* v, void* out, float* state_out,
                      int B, int H, int N, int d, int in_dt, int out_dt, float eps,
                      hipStream_t stream) {
  return forward(q, k, v, nullptr, false, false, out, state_out, B, H, N, N > 0 ? N : 1, d, in_dt, out_dt,
                 eps, nullptr, stream);
}

int la_global_forward_ex(const void* q, const void* k, const void* v, void* out, float* state_out,
                         int B, int H, int N, int d, int in_dt, int out_dt, float eps,
                         const la_launch_opts* opts, hipStream_t stream) {
  return forward(q, k, v, nullptr, false, false, out, state_out, B, H, N, N > 0 ? N : 1, d, in_dt, out_dt,
                 eps, opts, stream);
}

int la_blockcausal_forward(const void* q, const void* k, const void* v, const float* state_in,
                           void* out, float* states, int B, int H, int N, int T, int d, int in_dt,
                           int out_dt, float eps, hipStream_t stream) {
  return forward(q, k, v, state_in, false, true, out, states, B, H, N, T, d, in_dt, out_dt, eps, nullptr,
                 stream);
}

int la_blockcausal_forward_ex(const void* q, const void* k, const void* v, const float* state_in,
                              void* out, float* states, int B, int H, int N, int T, int d,
                              int in_dt, int out_dt, float eps, const la_launch_opts* opts,
                              hipStream_t stream) {
  return forward(q, k, v, state_in, false, true, out, states, B, H, N, T, d, in_dt, out_dt, eps, opts,
                 stream);
}

int la_chunk_forward_rope(const void* q, const void* k, const void* v, const float* state_in,
                          void* out, float* state_out, int B, int H, int L, int d, int in_dt,
                          int out_dt, float eps, int frame0, int grid_h, int grid_w, float theta,
                          hipStream_t stream) {
  const la::RopeGrid g = rope_grid(frame0, grid_h, grid_w, theta);
  return forward(q, k, v, state_in, true, false, out, state_out, B, H, L, L > 0 ? L : 1, d,
                 in_dt, out_dt, eps, nullptr, stream, &g);
}

int la_global_forward_rope(const void* q, const void* k, const void* v, void* out,
                           float* state_out, int B, int H, int N, int d, int in_dt, int out_dt,
                           float eps, int frame0, int grid_h, int grid_w, float theta,
                           hipStream_t stream) {
  const la::RopeGrid g = rope_grid(frame0, grid_h, grid_w, theta);
  return forward(q, k, v, nullptr, false, false, out, state_out, B, H, N, N > 0 ? N : 1, d,
                 in_dt, out_dt, eps, nullptr, stream, &g);
}

int la_blockcausal_forward_rope(const void* q, const void* k, const void* v,
                                const float* state_in, void* out, float* states, int B, int H,
                                int N, int T, int d, int in_dt, int out_dt, float eps, int frame0,
                                int grid_h, int grid_w, float theta, hipStream_t stream) {
  const la::RopeGrid g = rope_grid(frame0, grid_h, grid_w, theta);
  return forward(q, k, v, state_in, false, true, out, states, B, H, N, T, d, in_dt, out_dt, eps,
                 nullptr, stream, &g);
}

int la_blockcausal_forward_rope_ex(const void* q, const void* k, const void* v,
                                   const float* state_in, void* out, float* states, int B, int H,
                                   int N, int T, int d, int in_dt, int out_dt, float eps,
                                   int frame0, int grid_h, int grid_w, float theta,
                                   const la_launch_opts* opts, hipStream_t stream) {
  const la::RopeGrid g = rope_grid(frame0, grid_h, grid_w, theta);
  return forward(q, k, v, state_in, false, true, out, states, B, H, N, T, d, in_dt, out_dt, eps,
                 opts, stream, &g);
}

int la_plan(int B, int H, int L, int d, int in_dt, int out_dt, int kv_splits_request,
            int readout_workgroups_request, int* kv_splits, int* readout_workgroups) {
  int rc = check_shape(B, H, L, d, in_dt, out_dt);
  if (rc != LA_OK) return rc;
  if ((rc = check_sizes(B, H, L, L > 0 ? L : 1, d)) != LA_OK) return rc;
  if (kv_splits == nullptr || readout_workgroups == nullptr) return LA_E_INVAL;
  const Plan p = make_plan(B, H, L, L > 0 ? L : 1, d, in_dt, out_dt, kv_splits_request,
                           readout_workgroups_request);
  *kv_splits = p.nblk == 0 ? 0 : p.splits;
  *readout_workgroups = p.readout_wgs;
  return LA_OK;
}

int la_backward_workspace_size(int B, int H, int N, int T, int d, int in_dt, size_t* bytes) {
  int rc = check_shape(B, H, N, d, in_dt, LA_F32);
  if (rc != LA_OK) return rc;
  if (T <= 0 || bytes == nullptr) return LA_E_INVAL;
  if ((rc = check_sizes(B, H, N, T, d)) != LA_OK) return rc;
  const BwdPlan p = N == 0 ? make_bwd_plan(B, H, 1, 1, d, in_dt, 1, 1, SIZE_MAX)
                           : make_bwd_plan(B, H, N, T, d, in_dt, 0, 0, SIZE_MAX);
  *bytes = p.ws_bytes;
  return LA_OK;
}

int la_backward_stream_count(int B, int H, int N, int T, int d, int in_dt, int rotary,
                             int* count) {
  int rc = check_shape(B, H, N, d, in_dt, LA_F32);
  if (rc != LA_OK) return rc;
  if (T <= 0 || count == nullptr) return LA_E_INVAL;
  if ((rc = check_sizes(B, H, N, T, d)) != LA_OK) return rc;
  *count = bwd_two_streams(B, H, N, d, in_dt, rotary != 0) ? 2 : 1;
  return LA_OK;
}

int la_backward_plan(int B, int H, int N, int T, int d, int in_dt, int rotary,
                     int query_splits_request, int key_workgroups_request,
                     size_t workspace_bytes, la_backward_shape* shape) {
  int rc = check_shape(B, H, N, d, in_dt, LA_F32);
  if (rc != LA_OK) return rc;
  if (T <= 0 || shape == nullptr || query_splits_request < 0 || key_workgroups_request < 0)
    return LA_E_INVAL;
  if ((rc = check_sizes(B, H, N, T, d)) != LA_OK) return rc;
  if (rotary != 0 && N >= kRopeMaxTokens - 64) return LA_E_INVAL;  // as check_rope
  *shape = la_backward_shape{};
  if (N == 0) return LA_OK;
  const BwdPlan p = make_bwd_plan(B, H, N, T, d, in_dt, query_splits_request,
                                  key_workgroups_request,
                                  workspace_bytes == 0 ? SIZE_MAX : workspace_bytes,
                                  rotary != 0);
  if (workspace_bytes != 0 && p.ws_bytes > workspace_bytes) return LA_E_INVAL;
  // float32 kernels launch one workgroup per (b, h, block, split or item)
  const long long pairs = static_cast<long long>(B) * H * p.nblk;
  const bool bf = in_dt == LA_BF16;
  shape->blocks = p.nblk;
  shape->query_splits = p.qs;
  shape->query_workgroups = bf ? p.qgrid : static_cast<int>(pairs * p.qs);
  shape->key_items = p.ksweep ? 0 : p.ks;
  shape->key_workgroups = p.ksweep || bf ? p.kgrid : static_cast<int>(pairs * p.ks);
  shape->key_sweep_units = p.ksweep ? p.kupb : 0;
  return LA_OK;
}

int la_blockcausal_backward(const void* q, const void* k, const void* v, const float* states,
                            const void* dout, const float* dstates, void* dq, void* dk, void* dv,
                            float* dstate_in, int B, int H, int N, int T, int d, int in_dt,
                            int grad_dt, float eps, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return backward(q, k, v, states, dout, dstates, dq, dk, dv, dstate_in, B, H, N, T, d, in_dt,
                  grad_dt, eps, workspace, workspace_bytes, false, nullptr, stream);
}

int la_blockcausal_backward_ex(const void* q, const void* k, const void* v, const float* states,
                               const void* dout, const float* dstates, void* dq, void* dk,
                               void* dv, float* dstate_in, int B, int H, int N, int T, int d,
                               int in_dt, int grad_dt, float eps, void* workspace,
                               size_t workspace_bytes, const la_launch_opts* opts,
                               hipStream_t stream) {
  return backward(q, k, v, states, dout, dstates, dq, dk, dv, dstate_in, B, H, N, T, d, in_dt,
                  grad_dt, eps, workspace, workspace_bytes, false, opts, stream);
}

int la_blockcausal_backward_noalloc(const void* q, const void* k, const void* v,
                                    const float* states, const void* dout, const float* dstates,
                                    void* dq, void* dk, void* dv, float* dstate_in, int B, int H,
                                    int N, int T, int d, int in_dt, int grad_dt, float eps,
                                    hipStream_t stream) {
  return backward(q, k, v, states, dout, dstates, dq, dk, dv, dstate_in, B, H, N, T, d, in_dt,
                  grad_dt, eps, nullptr, 0, false, nullptr, stream, nullptr, true);
}

int la_chunk_backward(const void* q, const void* k, const void* v, const float* state_out,
                      const void* dout, const float* dstate_out, void* dq, void* dk, void* dv,
                      float* dstate_in, int B, int H, int L, int d, int in_dt, int grad_dt,
                      float eps, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (state_out == nullptr) return LA_E_INVAL;
  return backward(q, k, v, state_out, dout, dstate_out, dq, dk, dv, dstate_in, B, H, L,
                  L > 0 ? L : 1, d, in_dt, grad_dt, eps, workspace, workspace_bytes, L == 0,
                  nullptr, stream);
}

int la_chunk_backward_rope(const void* q, const void* k, const void* v, const float* state_out,
                           const void* dout, const float* dstate_out, void* dq, void* dk,
                           void* dv, float* dstate_in, int B, int H, int L, int d, int in_dt,
                           int grad_dt, float eps, void* workspace, size_t workspace_bytes,
                           int frame0, int grid_h, int grid_w, float theta, hipStream_t stream) {
  if (state_out == nullptr) return LA_E_INVAL;
  const la::RopeGrid g = rope_grid(frame0, grid_h, grid_w, theta);
  return backward(q, k, v, state_out, dout, dstate_out, dq, dk, dv, dstate_in, B, H, L,
                  L > 0 ? L : 1, d, in_dt, grad_dt, eps, workspace, workspace_bytes, L == 0,
                  nullptr, stream, &g);
}

int la_global_backward_rope(const void* q, const void* k, const void* v, const float* state,
                            const void* dout, void* dq, void* dk, void* dv, int B, int H, int N,
                            int d, int in_dt, int grad_dt, float eps, void* workspace,
                            size_t workspace_bytes, int frame0, int grid_h, int grid_w,
                            float theta, hipStream_t stream) {
  const la::RopeGrid g = rope_grid(frame0, grid_h, grid_w, theta);
  return backward(q, k, v, state, dout, nullptr, dq, dk, dv, nullptr, B, H, N, N > 0 ? N : 1, d,
                  in_dt, grad_dt, eps, workspace, workspace_bytes, false, nullptr, stream, &g);
}

int la_global_backward(const void* q, const void* k, const void* v, const float* state,
                       const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                       int in_dt, int grad_dt, float eps, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return backward(q, k, v, state, dout, nullptr, dq, dk, dv, nullptr, B, H, N, N > 0 ? N : 1, d,
                  in_dt, grad_dt, eps, workspace, workspace_bytes, false, nullptr, stream);
}

int la_blockcausal_backward_rope(const void* q, const void* k, const void* v,
                                 const float* states, const void* dout, const float* dstates,
                                 void* dq, void* dk, void* dv, float* dstate_in, int B, int H,
                                 int N, int T, int d, int in_dt, int grad_dt, float eps,
                                 void* workspace, size_t workspace_bytes, int frame0, int grid_h,
                                 int grid_w, float theta, hipStream_t stream) {
  const la::RopeGrid g = rope_grid(frame0, grid_h, grid_w, theta);
  return backward(q, k, v, states, dout, dstates, dq, dk, dv, dstate_in, B, H, N, T, d, in_dt,
                  grad_dt, eps, workspace, workspace_bytes, false, nullptr, stream, &g);
}

int la_blockcausal_backward_rope_ex(const void* q, const void* k, const void* v,
                                    const float* states, const void* dout, const float* dstates,
                                    void* dq, void* dk, void* dv, float* dstate_in, int B, int H,
                                    int N, int T, int d, int in_dt, int grad_dt, float eps,
                                    void* workspace, size_t workspace_bytes, int frame0,
                                    int grid_h, int grid_w, float theta,
                                    const la_launch_opts* opts, hipStream_t stream) {
  const la::RopeGrid g = rope_grid(frame0, grid_h, grid_w, theta);
  return backward(q, k, v, states, dout, dstates, dq, dk, dv, dstate_in, B, H, N, T, d, in_dt,
                  grad_dt, eps, workspace, workspace_bytes, false, opts, stream, &g);
}

int la_temporal_conv_chunk(const void* x, const void* cache_in, const float* weight,
                           const float* bias, void* y, void* cache_out, int B, int F, int P, int C,
                           int x_dt, int y_dt, hipStream_t stream) {
  return temporal_conv(x, cache_in, weight, bias, y, cache_out, B, F, F > 0 ? F : 1, P, C, x_dt,
                       y_dt, stream);
}

int la_temporal_conv_blockcausal(const void* x, const void* cache_in, const float* weight,
                                 const float* bias, void* y, void* cache_out, int B, int F, int Tf,
                                 int P, int C, int x_dt, int y_dt, hipStream_t stream) {
  return temporal_conv(x, cache_in, weight, bias, y, cache_out, B, F, Tf, P, C, x_dt, y_dt, stream);
}

const char* la_status_string(int status) {
  switch (status) {
    case LA_OK: return "ok";
    case LA_E_INVAL: return "invalid argument";
    case LA_E_UNSUPPORTED: return "unsupported head dimension or dtype";
    case LA_E_ALIGN: return "pointer not 16-byte aligned";
    case LA_E_ALIAS: return "illegal buffer overlap";
    case LA_E_HIP: return "HIP launch error";
    case LA_E_SCRATCH: return "needs more scratch than the static device buffer holds";
    default: return "unknown status";
  }
}

int la_abi_version(void) { return kAbiVersion; }

}  // extern "C"
