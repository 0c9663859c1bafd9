// Masked embedding lookup, its scatter-add backward, and the sampled-softmax
// candidate builder.
//
// Lookup ("Vocabulary shards: look up locally and normalize globally", ¶1-2):
// the shard owning an ID is found first (owner = ID div S for IDs in
// [0, V_real)), the row is read from that shard's slice at the local index,
// and the table is never addressed with an ID that failed the test. Output
// rows are copied (selected), so they are bit-exact with the table.
//
// Backward (same page, ¶2): repeated IDs add into their one owned row.
// Deterministic, one writer per row, no atomics on the table:
//   1. the valid tokens are sorted by (ID, token): up to 32768 tokens are cut
//      into runs of 1024 that workgroups radix-sort by ID in LDS, then each
//      workgroup places its run by ranking its IDs in all runs (two launches);
//      larger inputs use block-local LDS sorts, per-block ID counts and scans;
//   2. one launch sums the dout rows of each ID (a run of the sorted list)
//      and writes its row of dW once: an ID with fewer than kSegLong tokens
//      belongs to the chunk of kSegC sorted positions where its run starts,
//      and that chunk's wave sums it in sorted (= token) order; an ID with
//      kSegLong tokens or more is split by columns over many workgroups, each
//      of which sums its column slice over the whole run in a fixed order. No
//      partial sums leave a workgroup.
#include "vce_device.hpp"
#include "vce_internal.hpp"

namespace vce {

constexpr int kScanThreads = 256;
constexpr int kScanPerThread = 16;
constexpr int kScanBlock = kScanThreads * kScanPerThread;  // 4096 values per block
constexpr int kSegC = 16;                                  // sorted positions per chunk
constexpr int kSegBatch = 16;                              // dout rows in flight per lane
constexpr int kSegCols = 256;                              // dW columns per wave (64 lanes x 4)
constexpr int kRun = 1024;                                 // tokens per sorted run (one workgroup)
constexpr int kRunMaxRuns = 32;                            // runs the merge holds in LDS
constexpr int kPlanDigit = 6;                              // ID bits per radix pass
constexpr int kSortBlock = 1024;                           // tokens per local sort
constexpr int kSortThreads = 512;
constexpr int kSegLong = 64;     // tokens of an ID from which its sum is split by columns
constexpr int kLongCols = 64;    // columns per long-ID item (16 lanes x 4)
constexpr int kLongBatch = 16;   // dout rows in flight per lane of a long-ID item
constexpr int kLongWGs = 1024;   // workgroups that take the long-ID items

// ------------------------------------------------------------------ planning

int64_t scan_blocks(int64_t n) { return cdiv(n < 1 ? 1 : n, kScanBlock); }

static int32_t bit_width(int64_t x) {
  int32_t b = 0;
  while (x > 0) {
    ++b;
    x >>= 1;
  }
  return b;
}

EmbBwdPlan plan_emb_bwd(int64_t T, int64_t H, int64_t V_real, void* ws) {
  EmbBwdPlan p{};
  const int64_t Tp = T < 1 ? 1 : T;
  p.vbits = bit_width(V_real);
  // runs of kRun tokens sorted by workgroups, then merged (IDs < V_real <
  // 2^vbits stay below the all-ones value that marks tokens without a valid ID)
  p.nruns = cdiv(Tp, kRun);
  p.runs = p.nruns <= kRunMaxRuns;
  p.nblocks = cdiv(Tp, kSortBlock);
  p.nchunks = cdiv(Tp, kSegC);
  p.nslices = cdiv(H, kSegCols);
  p.scan_blocks = scan_blocks(V_real);
  Carve c(ws);
  if (!p.runs) {
    p.bcnt = c.take<int32_t>(static_cast<size_t>(p.nblocks * V_real));
    p.counts = c.take<int32_t>(static_cast<size_t>(V_real));
    p.offs = c.take<int32_t>(static_cast<size_t>(V_real + 1));
    p.lkey = c.take<uint64_t>(static_cast<size_t>(p.nblocks * kSortBlock));
    p.lrank = c.take<int32_t>(static_cast<size_t>(p.nblocks * kSortBlock));
    p.scan_tmp = c.take<int32_t>(static_cast<size_t>(p.scan_blocks + 1));
  } else {
    p.n_sorted = c.take<int32_t>(1);
    p.rid = c.take<uint32_t>(static_cast<size_t>(p.nruns * kRun));
    p.rtok = c.take<int32_t>(static_cast<size_t>(p.nruns * kRun));
    p.rvalid = c.take<int32_t>(static_cast<size_t>(p.nruns));
  }
  p.sorted = c.take<int32_t>(static_cast<size_t>(Tp));
  p.skey = c.take<int32_t>(static_cast<size_t>(Tp));
  p.chunk_start = c.take<int32_t>(static_cast<size_t>(p.nchunks));
  p.chunk_end = c.take<int32_t>(static_cast<size_t>(p.nchunks));
  p.long_runs = c.take<int32_t>(static_cast<size_t>(p.nchunks * 4));
  p.n_long = c.take<int32_t>(1);
  if (p.offs) p.n_sorted = p.offs + V_real;
  // long IDs: at most Tp / kSegLong of them, each cut into cdiv(H, kLongCols) items
  const int64_t long_items = (Tp / kSegLong) * cdiv(H, kLongCols);
  p.long_wgs = long_items < kLongWGs ? long_items : kLongWGs;
  p.bytes = c.used;
  return p;
}

CandPlan plan_cand(int64_t T, int64_t V, void* ws) {
  (void)T;
  CandPlan p{};
  p.scan_blocks_v = scan_blocks(V);
  Carve c(ws);
  p.flags = c.take<int32_t>(static_cast<size_t>(V));
  p.uidx = c.take<int32_t>(static_cast<size_t>(V + 1));
  p.notin = c.take<int32_t>(static_cast<size_t>(V));
  p.nidx = c.take<int32_t>(static_cast<size_t>(V + 1));
  p.scan_tmp = c.take<int32_t>(static_cast<size_t>(p.scan_blocks_v + 1));
  p.bytes = c.used;
  return p;
}

// ------------------------------------------------------------------ lookup

// kRowsPerWave output rows per wave, in 16-byte pieces: every load of the
// wave's rows is in flight before the first store. row_bytes is a multiple
// of 16. Workgroup 0 also counts the IDs outside [0, V_real) over all tokens
// and writes the count (a plain store: no counter to clear beforehand).
constexpr int kRowsPerWave = 1;
__global__ __launch_bounds__(256) void k_vemb_fwd(const int32_t* __restrict__ ids,
                                                  const char* __restrict__ W, int64_t T,
                                                  int64_t row_bytes, int64_t V_real,
                                                  const SegTable sg, char* __restrict__ out,
                                                  int32_t* n_bad) {
  constexpr int U = 8;  // pieces per lane and row held at once
  constexpr int RW = kRowsPerWave;
  const int lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && n_bad) {
    __shared__ int32_t cnt[4];
    // 16 reads in flight per lane: with one at a time this workgroup was the
    // launch's last to finish
    constexpr int UB = 16;
    int32_t bad = 0;
    for (int64_t b0 = 0; b0 < T; b0 += 256 * UB) {
      int32_t idv[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int64_t t = b0 + u * 256 + threadIdx.x;
        idv[u] = t < T ? ids[t] : 0;
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int64_t t = b0 + u * 256 + threadIdx.x;
        bad += (t < T && (idv[u] < 0 || idv[u] >= V_real)) ? 1 : 0;
      }
    }
    for (int o = 32; o > 0; o >>= 1) bad += __shfl_xor(bad, o);
    if (lane == 0) cnt[threadIdx.x >> 6] = bad;
    __syncthreads();
    if (threadIdx.x == 0) *n_bad = cnt[0] + cnt[1] + cnt[2] + cnt[3];
  }
  const int64_t t0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * RW;
  if (t0 >= T) return;
  const int64_t nvec = row_bytes >> 4;
  const u32x4* src[RW];
  u32x4* dst[RW];
  bool owned[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int64_t t = min(t0 + r, T - 1);
    const int64_t id = ids[t];
    // owner test, then the local index within the owner's slice
    owned[r] = (t0 + r < T) && (id >= 0) && (id < V_real);
    const int k = owned[r] ? shard_of_row(sg, id) : 0;
    const int64_t local = owned[r] ? id - sg.row[k] : 0;
    src[r] = reinterpret_cast<const u32x4*>(W + (sg.row[k] + local) * row_bytes);
    dst[r] = reinterpret_cast<u32x4*>(out + t * row_bytes);
  }
  for (int64_t c0 = 0; c0 < nvec; c0 += 64 * U) {
    u32x4 v[RW][U];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + lane + 64 * u;
        v[r][u] = (owned[r] && c < nvec) ? src[r][c] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + lane + 64 * u;
        if (t0 + r < T && c < nvec) {
          __builtin_nontemporal_store(v[r][u], dst[r] + c);
        }
      }
  }
}

__global__ void k_zero_i32(int32_t* p) {
  if (threadIdx.x == 0) *p = 0;
}

// out[t] = map[in[t]] for in[t] in [0, V_real); any other value passes through
// (explicitly mapped class ownership: class -> physical row, or back).
__global__ __launch_bounds__(256) void k_remap(const int32_t* __restrict__ in, int64_t T,
                                               const int32_t* __restrict__ map, int64_t V_real,
                                               int32_t* __restrict__ out) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  const int64_t v = in[t];
  out[t] = (v >= 0 && v < V_real) ? map[v] : static_cast<int32_t>(v);
}

hipError_t run_remap(const int32_t* in, int64_t T, const int32_t* map, int64_t V_real,
                     int32_t* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_remap, dim3(static_cast<uint32_t>(cdiv(T, 256))), dim3(256), 0, s, in, T,
                     map, V_real, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ hashed n-grams

// The SplitMix64 output finaliser (Steele, Lea and Flood, OOPSLA 2014).
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <typename E>
struct Piece;  // one 16-byte piece of a row, widened to float
template <>
struct Piece<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const u32x4& v, float (&f)[8]) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
  }
  __device__ static u32x4 store(const float (&f)[8]) {
    return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
  }
};
template <>
struct Piece<float> {
  static constexpr int N = 4;
  __device__ static void load(const u32x4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static u32x4 store(const float (&f)[4]) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
};

// Input embedding of the Over-Tokenized Transformer's input side ("Sampled
// Softmax with Over-Tokenized Transformer", Setup): one wave per token t
//   x[t] = E[id_t] + E2[row2(t)] + E3[row3(t)]
// where row_n(t) is mix64(key) mod rows_n for the n-gram ending at t (key =
// its token IDs in base V_real, oldest first), present only when t >= n-1 and
// all n IDs are valid; a missing part adds nothing. Every table is read by
// owner shard and local index (contiguous equal shards). The three pieces
// are added in float32 in that order and the sum is stored in the table
// type (bf16 rounded to nearest-even). row2 / row3 (-1 if missing) are
// written for the backward. Workgroup 0 counts invalid token IDs.
template <typename E>
__global__ __launch_bounds__(256) void k_ngram_fwd(
    const int32_t* __restrict__ ids, const char* __restrict__ E0, const char* __restrict__ E2,
    const char* __restrict__ E3, int64_t T, int64_t row_bytes, int64_t V_real, int64_t S0,
    int64_t rows2, int64_t S2, int64_t rows3, int64_t S3, char* __restrict__ out,
    int32_t* __restrict__ ids2, int32_t* __restrict__ ids3, int32_t* n_bad) {
  constexpr int U = 8;  // pieces per lane and table held at once
  const int lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && n_bad) {
    __shared__ int32_t cnt[4];
    // 16 reads in flight per lane: with one at a time this workgroup was the
    // launch's last to finish
    constexpr int UB = 16;
    int32_t bad = 0;
    for (int64_t b0 = 0; b0 < T; b0 += 256 * UB) {
      int32_t idv[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int64_t t = b0 + u * 256 + threadIdx.x;
        idv[u] = t < T ? ids[t] : 0;
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int64_t t = b0 + u * 256 + threadIdx.x;
        bad += (t < T && (idv[u] < 0 || idv[u] >= V_real)) ? 1 : 0;
      }
    }
    for (int o = 32; o > 0; o >>= 1) bad += __shfl_xor(bad, o);
    if (lane == 0) cnt[threadIdx.x >> 6] = bad;
    __syncthreads();
    if (threadIdx.x == 0) *n_bad = cnt[0] + cnt[1] + cnt[2] + cnt[3];
  }
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t a = ids[t];
  const int64_t b = t >= 1 ? ids[t - 1] : -1;
  const int64_t c = t >= 2 ? ids[t - 2] : -1;
  const bool oka = a >= 0 && a < V_real, okb = b >= 0 && b < V_real, okc = c >= 0 && c < V_real;
  const uint64_t V = static_cast<uint64_t>(V_real);
  int64_t r2 = -1, r3 = -1;
  if (oka && okb) r2 = static_cast<int64_t>(mix64(static_cast<uint64_t>(b) * V + a) % rows2);
  if (oka && okb && okc)
    r3 = static_cast<int64_t>(mix64((static_cast<uint64_t>(c) * V + b) * V + a) % rows3);
  if (lane == 0) {
    ids2[t] = static_cast<int32_t>(r2);
    ids3[t] = static_cast<int32_t>(r3);
  }
  // owner shard, then the local row inside its slice, for each table
  auto row_ptr = [&](const char* base, int64_t r, int64_t S) -> const u32x4* {
    const int64_t k = r / S;
    return reinterpret_cast<const u32x4*>(base + (k * S + (r - k * S)) * row_bytes);
  };
  const u32x4* p0 = oka ? row_ptr(E0, a, S0) : nullptr;
  const u32x4* p2 = r2 >= 0 ? row_ptr(E2, r2, S2) : nullptr;
  const u32x4* p3 = r3 >= 0 ? row_ptr(E3, r3, S3) : nullptr;
  u32x4* dst = reinterpret_cast<u32x4*>(out + t * row_bytes);
  const int64_t nvec = row_bytes >> 4;
  constexpr u32x4 kZero = {0u, 0u, 0u, 0u};
  for (int64_t c0 = 0; c0 < nvec; c0 += 64 * U) {
    u32x4 v0[U], v2[U], v3[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t cc = c0 + lane + 64 * u;
      const bool in = cc < nvec;
      v0[u] = (in && p0) ? p0[cc] : kZero;
      v2[u] = (in && p2) ? p2[cc] : kZero;
      v3[u] = (in && p3) ? p3[cc] : kZero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t cc = c0 + lane + 64 * u;
      if (cc >= nvec) continue;
      float f0[Piece<E>::N], f2[Piece<E>::N], f3[Piece<E>::N];
      Piece<E>::load(v0[u], f0);
      Piece<E>::load(v2[u], f2);
      Piece<E>::load(v3[u], f3);
#pragma unroll
      for (int i = 0; i < Piece<E>::N; ++i) f0[i] = (f0[i] + f2[i]) + f3[i];
      __builtin_nontemporal_store(Piece<E>::store(f0), dst + cc);
    }
  }
}

hipError_t run_ngram_fwd(const int32_t* ids, const void* E0, const void* E2, const void* E3,
                         int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int64_t rows2,
                         int64_t rows3, int32_t n, bool bf16, void* out, int32_t* ids2,
                         int32_t* ids3, int32_t* n_bad, hipStream_t s) {
  if (T == 0) {
    if (!n_bad) return hipSuccess;
    hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(64), 0, s, n_bad);
    return hipGetLastError();
  }
  const int64_t row_bytes = H * (bf16 ? 2 : 4);
  const dim3 grid(static_cast<uint32_t>(cdiv(T, 4)));
  if (bf16)
    hipLaunchKernelGGL(k_ngram_fwd<uint16_t>, grid, dim3(256), 0, s, ids,
                       static_cast<const char*>(E0), static_cast<const char*>(E2),
                       static_cast<const char*>(E3), T, row_bytes, V_real, V_pad / n, rows2,
                       rows2 / n, rows3, rows3 / n, static_cast<char*>(out), ids2, ids3, n_bad);
  else
    hipLaunchKernelGGL(k_ngram_fwd<float>, grid, dim3(256), 0, s, ids,
                       static_cast<const char*>(E0), static_cast<const char*>(E2),
                       static_cast<const char*>(E3), T, row_bytes, V_real, V_pad / n, rows2,
                       rows2 / n, rows3, rows3 / n, static_cast<char*>(out), ids2, ids3, n_bad);
  return hipGetLastError();
}


// ------------------------------------------------------------------ scan

__global__ __launch_bounds__(kScanThreads) void k_fill_i32(int32_t* __restrict__ p, int64_t n,
                                                           int32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kScanThreads + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void k_fill_f4(float4* __restrict__ p, int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Block-local exclusive scan of 4096 values; block totals to tmp[block].
__global__ __launch_bounds__(kScanThreads) void k_scan_local(const int32_t* __restrict__ x,
                                                             int64_t n, int32_t* __restrict__ y,
                                                             int32_t* __restrict__ tmp) {
  __shared__ int32_t s[kScanThreads];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanBlock + threadIdx.x * kScanPerThread;
  int32_t v[kScanPerThread];
  int32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kScanPerThread; ++i) {
    v[i] = (base + i < n) ? x[base + i] : 0;
    sum += v[i];
  }
  s[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t a = (static_cast<int>(threadIdx.x) >= off) ? s[threadIdx.x - off] : 0;
    __syncthreads();
    s[threadIdx.x] += a;
    __syncthreads();
  }
  int32_t run = s[threadIdx.x] - sum;  // exclusive prefix of this thread
#pragma unroll
  for (int i = 0; i < kScanPerThread; ++i) {
    if (base + i < n) y[base + i] = run;
    run += v[i];
  }
  if (threadIdx.x == kScanThreads - 1) tmp[blockIdx.x] = s[threadIdx.x];
}

// Exclusive scan of the block totals (one block, sequential per thread group).
__global__ __launch_bounds__(kScanThreads) void k_scan_top(int32_t* __restrict__ tmp,
                                                           int64_t nb) {
  __shared__ int32_t s[kScanThreads];
  // each thread owns a contiguous run of ceil(nb / 256) totals
  const int64_t per = (nb + kScanThreads - 1) / kScanThreads;
  const int64_t b0 = threadIdx.x * per;
  int32_t sum = 0;
  for (int64_t i = b0; i < b0 + per && i < nb; ++i) sum += tmp[i];
  s[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t a = (static_cast<int>(threadIdx.x) >= off) ? s[threadIdx.x - off] : 0;
    __syncthreads();
    s[threadIdx.x] += a;
    __syncthreads();
  }
  int32_t run = s[threadIdx.x] - sum;
  for (int64_t i = b0; i < b0 + per && i < nb; ++i) {
    const int32_t v = tmp[i];
    tmp[i] = run;
    run += v;
  }
  if (threadIdx.x == kScanThreads - 1) tmp[nb] = s[threadIdx.x];
}

// y[i] += tmp[block]; y[n] = total; optional copy
__global__ __launch_bounds__(kScanThreads) void k_scan_add(int32_t* __restrict__ y, int64_t n,
                                                           int32_t* __restrict__ y_copy,
                                                           const int32_t* __restrict__ tmp,
                                                           int64_t nb) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kScanThreads + threadIdx.x;
  if (i < n) {
    const int32_t v = y[i] + tmp[i / kScanBlock];
    y[i] = v;
    if (y_copy) y_copy[i] = v;
  } else if (i == n) {
    y[n] = tmp[nb];
    if (y_copy) y_copy[n] = tmp[nb];
  }
}

hipError_t run_scan(const int32_t* x, int64_t n, int32_t* y, int32_t* y_copy, int32_t* tmp,
                    hipStream_t s) {
  const int64_t nb = scan_blocks(n);
  hipLaunchKernelGGL(k_scan_local, dim3(static_cast<uint32_t>(nb)), dim3(kScanThreads), 0, s, x, n,
                     y, tmp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(kScanThreads), 0, s, tmp, nb);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_scan_add, dim3(static_cast<uint32_t>(cdiv(n + 1, kScanThreads))),
                     dim3(kScanThreads), 0, s, y, n, y_copy, tmp, nb);
  return hipGetLastError();
}

// ------------------------------------------------------------------ scatter-add

__global__ __launch_bounds__(256) void k_fill_i32x4(int4* __restrict__ p, int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) p[i] = make_int4(0, 0, 0, 0);
}

__device__ __forceinline__ int lds_lower_bound(const uint64_t* s, uint64_t key) {
  int lo = 0, hi = kSortBlock;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Block b sorts the keys (ID << 32 | token) of tokens [b*1024, (b+1)*1024) in
// LDS (bitonic network; tokens with an ID outside [0, V_real) sort last),
// writes the sorted keys, each token's rank among equal IDs of the block, and
// the block's count of every ID it holds into bcnt[b][ID].
__global__ __launch_bounds__(kSortThreads) void k_block_sort(const int32_t* __restrict__ ids,
                                                             int64_t T, int64_t V_real,
                                                             uint64_t* __restrict__ lkey,
                                                             int32_t* __restrict__ lrank,
                                                             int32_t* __restrict__ bcnt,
                                                             int32_t* __restrict__ n_long) {
  __shared__ uint64_t s[kSortBlock];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  if (b == 0 && tid == 0) *n_long = 0;  // k_chunk_starts appends the long IDs
  constexpr uint64_t kNone = ~0ull;
#pragma unroll
  for (int u = 0; u < kSortBlock / kSortThreads; ++u) {
    const int i = tid + u * kSortThreads;
    const int64_t t = b * kSortBlock + i;
    uint64_t key = kNone;
    if (t < T) {
      const int64_t id = ids[t];
      if (id >= 0 && id < V_real)
        key = (static_cast<uint64_t>(id) << 32) | static_cast<uint64_t>(t);
    }
    s[i] = key;
  }
  __syncthreads();
  for (int k = 2; k <= kSortBlock; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int i = ((tid & ~(j - 1)) << 1) | (tid & (j - 1));  // bit j of i is clear
      const int pj = i | j;
      const uint64_t a = s[i], c = s[pj];
      const bool up = (i & k) == 0;
      if ((a > c) == up) {
        s[i] = c;
        s[pj] = a;
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int u = 0; u < kSortBlock / kSortThreads; ++u) {
    const int i = tid + u * kSortThreads;
    const uint64_t key = s[i];
    int rank = 0;
    if (key != kNone) {
      const uint64_t id = key >> 32;
      const int lo = lds_lower_bound(s, id << 32);
      rank = i - lo;
      if (rank == 0) {
        const int hi = lds_lower_bound(s, (id + 1) << 32);
        bcnt[b * V_real + static_cast<int64_t>(id)] = hi - lo;
      }
    }
    lkey[b * kSortBlock + i] = key;
    lrank[b * kSortBlock + i] = rank;
  }
}

// Per ID: turn the per-block counts into per-block offsets (in block order)
// and the total count.
__global__ __launch_bounds__(256) void k_col_scan(int32_t* __restrict__ bcnt, int64_t nblocks,
                                                  int64_t V_real, int32_t* __restrict__ counts) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (v >= V_real) return;
  int32_t run = 0;
  for (int64_t b = 0; b < nblocks; ++b) {
    const int32_t c = bcnt[b * V_real + v];
    bcnt[b * V_real + v] = run;
    run += c;
  }
  counts[v] = run;
}

// sorted[offs[ID] + block offset + rank] = token: stable, one writer per slot
__global__ __launch_bounds__(256) void k_place_sorted(const uint64_t* __restrict__ lkey,
                                                      const int32_t* __restrict__ lrank,
                                                      const int32_t* __restrict__ bcnt,
                                                      const int32_t* __restrict__ offs,
                                                      int64_t n, int64_t V_real,
                                                      int32_t* __restrict__ sorted,
                                                      int32_t* __restrict__ skey) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const uint64_t key = lkey[i];
  if (key == ~0ull) return;
  const int64_t id = static_cast<int64_t>(key >> 32);
  const int64_t b = i / kSortBlock;
  const int64_t dst = offs[id] + bcnt[b * V_real + id] + lrank[i];
  sorted[dst] = static_cast<int32_t>(key & 0xFFFFFFFFu);
  skey[dst] = static_cast<int32_t>(id);
}

template <typename D>
__device__ __forceinline__ f32x4 load_row4(const D* row, int64_t col);
template <>
__device__ __forceinline__ f32x4 load_row4<float>(const float* row, int64_t col) {
  return *reinterpret_cast<const f32x4*>(row + col);
}
template <>
__device__ __forceinline__ f32x4 load_row4<uint16_t>(const uint16_t* row, int64_t col) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(row + col);
  f32x4 r;
  r.x = __uint_as_float(w.x << 16);
  r.y = __uint_as_float(w.x & 0xFFFF0000u);
  r.z = __uint_as_float(w.y << 16);
  r.w = __uint_as_float(w.y & 0xFFFF0000u);
  return r;
}

// ---------------------------------------------------------- one-workgroup sort

// Bits [0, 64) of a wave-wide mask: lanes whose value v equals this lane's
// (kPlanDigit-bit digits compared bit by bit through ballots).
__device__ __forceinline__ uint64_t match_digit(uint32_t d) {
  uint64_t eq = ~0ull;
#pragma unroll
  for (int b = 0; b < kPlanDigit; ++b) {
    // x: all ones where this lane's bit b is set; lanes that agree with it
    // on bit b are the set bits of ~(ballot ^ x)
    const uint32_t x32 = 0u - ((d >> b) & 1u);
    const uint64_t x = (static_cast<uint64_t>(x32) << 32) | x32;
    const uint64_t m = __ballot(x32 != 0u);
    eq &= ~(m ^ x);
  }
  return eq;
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele steps of
// 1, 2, 4 and 8 lanes within each row of 16 lanes (DPP row shifts; lanes
// shifted in from outside the row read 0), then the totals of the lower rows
// (lanes 15, 31 and 47) are added.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  int v = static_cast<int>(x);
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  v += (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
  return static_cast<uint32_t>(v);
}

// Sort of the tokens of one call by (ID, token), in two steps.
// k_run_sort: workgroup r sorts the run of tokens [r*kRun, (r+1)*kRun) by ID,
// stably (least-significant-digit radix passes of kPlanDigit ID bits; within
// a wave, lanes with the same digit are found bit by bit through ballots and
// ranked by lane; across waves, counts are scanned in (digit, wave) order).
// Tokens without a valid ID carry all bits set and end their run.
__global__ __launch_bounds__(kRun) void k_run_sort(const int32_t* __restrict__ ids, int64_t T,
                                                   int64_t V_real, int32_t vbits,
                                                   uint32_t* __restrict__ rid,
                                                   int32_t* __restrict__ rtok,
                                                   int32_t* __restrict__ rvalid,
                                                   int32_t* __restrict__ n_long) {
  constexpr int NW = kRun / 64;
  constexpr int ND = 1 << kPlanDigit;
  static_assert(NW * ND == kRun, "one thread per (wave, digit) count");
  __shared__ uint32_t kid[2][kRun];
  __shared__ int32_t ktok[2][kRun];
  __shared__ uint32_t wrun[NW][ND];
  __shared__ uint32_t wtot[NW];
  __shared__ int32_t s_n;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRun + tid;
  uint32_t id = ~0u;
  if (t < T) {
    const int64_t v = ids[t];
    if (v >= 0 && v < V_real) id = static_cast<uint32_t>(v);
  }
  if (tid == 0) s_n = 0;
  if (blockIdx.x == 0 && tid == 0) *n_long = 0;  // the merge appends the long IDs
  kid[0][tid] = id;
  ktok[0][tid] = static_cast<int32_t>(t);
  __syncthreads();
  const uint64_t vb = __ballot(id != ~0u);
  if (lane == 0) atomicAdd(&s_n, static_cast<int32_t>(__popcll(vb)));

  int src = 0;
  const int npass = (vbits + kPlanDigit - 1) / kPlanDigit;
  for (int pass = 0; pass < npass; ++pass) {
    const int shift = kPlanDigit * pass;
    wrun[w][lane] = 0u;  // this wave's counters; only this wave touches them until the barrier
    const uint32_t key = kid[src][tid];
    const int32_t tk = ktok[src][tid];
    const uint32_t d = (key >> shift) & (ND - 1);
    const uint64_t eq = match_digit(d);
    const uint32_t below = static_cast<uint32_t>(__popcll(eq & lt));
    if (below == 0) wrun[w][d] = static_cast<uint32_t>(__popcll(eq));
    __syncthreads();
    // exclusive scan of the counts in (digit, wave) order: thread i holds
    // digit i / NW, wave i % NW
    const int di = tid / NW, wi = tid % NW;
    const uint32_t v = wrun[wi][di];
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) wtot[w] = x;
    __syncthreads();
    uint32_t base = 0;  // all NW reads issued together (broadcasts)
#pragma unroll
    for (int k = 0; k < NW; ++k) base += k < w ? wtot[k] : 0u;
    wrun[wi][di] = base + x - v;  // every thread has read its count above
    __syncthreads();
    const uint32_t pos = wrun[w][d] + below;
    kid[src ^ 1][pos] = key;
    ktok[src ^ 1][pos] = tk;
    __syncthreads();
    src ^= 1;
  }
  const int64_t o = static_cast<int64_t>(blockIdx.x) * kRun + tid;
  rid[o] = kid[src][tid];
  rtok[o] = ktok[src][tid];
  if (tid == 0) rvalid[blockIdx.x] = s_n;
}

// Both bounds of x (< 2^31) in the runs k = q, q + 4, q + 8, ... below
// nruns (U slots): lt_k = #(IDs < x) and le_k = #(IDs <= x) among the run's
// kRun ascending IDs. Adds to off (le_k for k < r, lt_k for k > r), lt and le.
// The 2U binary searches advance together with no branches (a slot past
// nruns searches the last run and adds nothing), so the 2U LDS reads of a
// step are in flight at once.
template <int U>
__device__ __forceinline__ void run_bounds(const uint32_t* all, int nruns, int q, int r,
                                           uint32_t x, int32_t& off, int32_t& lt, int32_t& le) {
  const uint32_t* base[U];
  int32_t a[U], b[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = q + 4 * u;
    base[u] = all + (k < nruns ? k : nruns - 1) * kRun;
    a[u] = 0;
    b[u] = 0;
  }
#pragma unroll
  for (int step = kRun / 2; step > 0; step >>= 1) {
    uint32_t ya[U], yb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ya[u] = base[u][a[u] + step - 1];
      yb[u] = base[u][b[u] + step - 1];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] += ya[u] < x ? step : 0;
      b[u] += yb[u] <= x ? step : 0;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // a, b <= kRun - 1 here: element a (b) is the last one left to test
    const int k = q + 4 * u;
    const int32_t ra = a[u] + (base[u][a[u]] < x ? 1 : 0);
    const int32_t rb = b[u] + (base[u][b[u]] <= x ? 1 : 0);
    if (k < nruns) {
      lt += ra;
      le += rb;
      off += k < r ? rb : (k > r ? ra : 0);
    }
  }
}

// k_run_merge: a workgroup places kRankTok tokens of one run, four threads
// per token, each searching a quarter of the runs. With the runs' IDs in
// LDS, a token at index i of run r with ID v goes to
//   i + (tokens with ID <= v in runs before r) + (tokens with ID < v in runs after r),
// which is its rank in (ID, token) order, since run r holds tokens
// [r*kRun, (r+1)*kRun). The same searches give where v's tokens start and
// end in the sorted list: a token at a chunk's first position records them
// for its chunk, and the first token of an ID with at least kSegLong tokens
// appends the ID's (start, end) to the long list (in any order).
constexpr int kRankTok = 64;
constexpr int kMergeSplit = kRun / kRankTok;  // workgroups per run
static_assert(kRunMaxRuns <= 64, "one wave sums the run counts");
static_assert(kRunMaxRuns % 4 == 0, "four threads per token split the runs");
__global__ __launch_bounds__(4 * kRankTok) void k_run_merge(
    const uint32_t* __restrict__ rid, const int32_t* __restrict__ rtok,
    const int32_t* __restrict__ rvalid, int32_t nruns, int32_t* __restrict__ sorted,
    int32_t* __restrict__ skey, int32_t* __restrict__ n_sorted,
    int32_t* __restrict__ chunk_start, int32_t* __restrict__ chunk_end,
    int32_t* __restrict__ long_runs, int32_t* __restrict__ n_long, int32_t long_cap) {
  __shared__ __attribute__((aligned(16))) uint32_t all[kRunMaxRuns * kRun];
  constexpr int NT = 4 * kRankTok;
  const int tid = threadIdx.x;
  const int r = blockIdx.x / kMergeSplit;
  const int i = (blockIdx.x % kMergeSplit) * kRankTok + tid / 4;  // index in run r
  const int q = tid % 4;                                           // runs q, q+4, ...
  // nruns * kRun IDs: nruns * kRun / (4 * NT) 16-byte pieces per thread,
  // sixteen loads in flight
  const int32_t tk = rtok[r * kRun + i];  // loaded with the IDs, used at the end
  const u32x4* src = reinterpret_cast<const u32x4*>(rid);
  u32x4* dst = reinterpret_cast<u32x4*>(all);
  const int npieces = nruns * (kRun / 4);
  for (int p0 = 0; p0 < npieces; p0 += 16 * NT) {
    u32x4 x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (p0 + u * NT + tid < npieces) x[u] = src[p0 + u * NT + tid];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (p0 + u * NT + tid < npieces) dst[p0 + u * NT + tid] = x[u];
  }
  if (blockIdx.x == 0 && tid < 64) {  // nruns <= 64: one load per lane, one wave sum
    int32_t n = tid < nruns ? rvalid[tid] : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
    if (tid == 0) *n_sorted = n;
  }
  __syncthreads();
  const uint32_t v = all[r * kRun + i];
  if (v == ~0u) return;  // the same for the four threads of a token
  int32_t off = 0, lt = 0, le = 0;
  if (nruns <= kRunMaxRuns / 2)  // uniform
    run_bounds<kRunMaxRuns / 8>(all, nruns, q, r, v, off, lt, le);
  else
    run_bounds<kRunMaxRuns / 4>(all, nruns, q, r, v, off, lt, le);
  // sums over the four threads of the token (adjacent lanes)
#pragma unroll
  for (int o = 1; o < 4; o <<= 1) {
    off += __shfl_xor(off, o);
    lt += __shfl_xor(lt, o);
    le += __shfl_xor(le, o);
  }
  if (q != 0) return;
  const int32_t pos = i + off;
  sorted[pos] = tk;
  skey[pos] = static_cast<int32_t>(v);
  if (pos % kSegC == 0) {
    chunk_start[pos / kSegC] = lt;
    chunk_end[pos / kSegC] = le;
  }
  if (pos == lt && le - lt >= kSegLong) {
    const int32_t k = atomicAdd(n_long, 1);
    if (k < long_cap)  // at most (tokens / kSegLong) long IDs: always true
      reinterpret_cast<i32x4*>(long_runs)[k] = i32x4{lt, le, static_cast<int32_t>(v), 0};
  }
}

// General sort: where the tokens of the ID at every chunk's first position
// start and end in the sorted list; the chunk holding the first chunk start
// inside a long ID's run appends the ID to the long list.
__global__ __launch_bounds__(256) void k_chunk_starts(const int32_t* __restrict__ skey,
                                                      const int32_t* __restrict__ offs,
                                                      const int32_t* __restrict__ n_sorted,
                                                      int64_t nchunks,
                                                      int32_t* __restrict__ chunk_start,
                                                      int32_t* __restrict__ chunk_end,
                                                      int32_t* __restrict__ long_runs,
                                                      int32_t* __restrict__ n_long) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = *n_sorted;
  if (c >= nchunks || c * kSegC >= n) return;
  const int64_t id = skey[c * kSegC];
  const int32_t lt = offs[id], le = offs[id + 1];
  chunk_start[c] = lt;
  chunk_end[c] = le;
  if (le - lt >= kSegLong && lt > c * kSegC - kSegC) {
    const int32_t k = atomicAdd(n_long, 1);
    if (k < nchunks)  // at most (tokens / kSegLong) long IDs: always true
      reinterpret_cast<i32x4*>(long_runs)[k] = i32x4{lt, le, static_cast<int32_t>(id), 0};
  }
}

// ------------------------------------------------------------------ segment sums

// Long IDs: item j = (long ID j / nls, column slice j % nls) of kLongCols
// columns; the workgroups [0, long_wgs) take items wg, wg + long_wgs, ...
// kLongRowLanes row lanes (groups of kLongCols / 4 lanes, 4 columns per
// lane) each sum every kLongRowLanes-th token of the run in sorted order,
// kLongBatch rows in flight, the next batch's token indices loading behind
// them; the row lanes' sums are added in row-lane order through LDS and the
// slice of the ID's row is written (added to when accumulating) once.
constexpr int kLongLanesPerRow = kLongCols / 4;
constexpr int kLongRowLanes = 256 / kLongLanesPerRow;
template <typename D>
__device__ __forceinline__ void seg_long(int64_t wg, int64_t nwg, const int32_t* skey,
                                         const int32_t* sorted, const int32_t* long_runs,
                                         int32_t n_long, int32_t N, const D* dout, int64_t H,
                                         float* dW, int32_t accumulate,
                                         f32x4 (*red)[kLongLanesPerRow]) {
  const int rl = threadIdx.x / kLongLanesPerRow;  // row lane
  const int cl = threadIdx.x % kLongLanesPerRow;  // column lane
  const int64_t nls = (H + kLongCols - 1) / kLongCols;
  const int64_t items = static_cast<int64_t>(n_long) * nls;
  constexpr int STEP = kLongRowLanes * kLongBatch;  // positions per batch of the workgroup
  for (int64_t j = wg; j < items; j += nwg) {
    const int64_t k = j / nls;
    // (first, end) lie in [0, N] with first < end; clamped all the same, so
    // that no read can leave the sorted list
    const i32x4 e = reinterpret_cast<const i32x4*>(long_runs)[k];
    const int32_t end = min(e.y, N);
    const int32_t first = max(0, min(e.x, end - 1));
    const int64_t col = (j % nls) * kLongCols + cl * 4;
    const bool active = col < H;
    const int64_t colc = active ? col : H - 4;  // a readable column; its sum is dropped
    // the row slice this item adds into, loaded now and used at the end
    f32x4* dst = reinterpret_cast<f32x4*>(dW + static_cast<int64_t>(e.z) * H + colc);
    f32x4 old = {0.f, 0.f, 0.f, 0.f};
    if (accumulate && threadIdx.x < kLongLanesPerRow) old = *dst;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int32_t tok[kLongBatch];
#pragma unroll
    for (int u = 0; u < kLongBatch; ++u)
      tok[u] = sorted[min(first + u * kLongRowLanes + rl, end - 1)];
    for (int32_t b0 = first; b0 < end; b0 += STEP) {
      f32x4 row[kLongBatch];
#pragma unroll
      for (int u = 0; u < kLongBatch; ++u)
        row[u] = load_row4<D>(dout + static_cast<int64_t>(tok[u]) * H, colc);
      if (b0 + STEP < end) {
#pragma unroll
        for (int u = 0; u < kLongBatch; ++u)
          tok[u] = sorted[min(b0 + STEP + u * kLongRowLanes + rl, end - 1)];
      }
#pragma unroll
      for (int u = 0; u < kLongBatch; ++u)
        if (b0 + u * kLongRowLanes + rl < end) acc += row[u];
    }
    red[rl][cl] = acc;
    __syncthreads();
    if (threadIdx.x < kLongLanesPerRow && active) {  // row lane 0: cl == threadIdx.x
      f32x4 tot = red[0][cl];
#pragma unroll
      for (int q = 1; q < kLongRowLanes; ++q) tot += red[q][cl];
      *dst = accumulate ? old + tot : tot;
    }
    __syncthreads();  // red is reused by the next item
  }
}

// The segment sums of every ID, one launch. Workgroups below long_wgs take
// the long IDs (seg_long); each other workgroup is a chunk of kSegC sorted
// positions and four 256-column slices of dW, one per wave. A chunk owns the
// IDs with fewer than kSegLong tokens whose run starts inside it, whole: from
// its first position (or the end of a run that came from before or is long)
// to the end of the last such run, which may reach past the chunk. Its wave
// sums each run in sorted (= token) order and writes (or adds into) the ID's
// row; run boundaries depend on the sorted IDs only, so every branch is
// uniform across the wave, and the dout rows of a batch and the dW rows its
// runs update are all in flight before the first add.
template <typename D>
__global__ __launch_bounds__(256) void k_seg_sums(const int32_t* __restrict__ skey,
                                                  const int32_t* __restrict__ sorted,
                                                  const int32_t* __restrict__ n_sorted,
                                                  const int32_t* __restrict__ chunk_start,
                                                  const int32_t* __restrict__ chunk_end,
                                                  const int32_t* __restrict__ long_runs,
                                                  const int32_t* __restrict__ n_long,
                                                  const D* __restrict__ dout, int64_t H,
                                                  int64_t nslices, int64_t nchunks,
                                                  int64_t long_wgs, float* __restrict__ dW,
                                                  int32_t accumulate) {
  __shared__ f32x4 red[kLongRowLanes][kLongLanesPerRow];
  if (static_cast<int64_t>(blockIdx.x) < long_wgs) {
    const int32_t nl = min(*n_long, static_cast<int32_t>(nchunks));
    seg_long<D>(blockIdx.x, long_wgs, skey, sorted, long_runs, nl, *n_sorted, dout, H, dW,
                accumulate, red);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t ngroups = (nslices + 3) / 4;
  const int64_t item = static_cast<int64_t>(blockIdx.x) - long_wgs;
  const int64_t c = item / ngroups;
  const int64_t slice = (item % ngroups) * 4 + (threadIdx.x >> 6);
  const int64_t N = *n_sorted;
  const int64_t p0 = c * kSegC;
  if (slice >= nslices || p0 >= N) return;
  // [pb, pe): whole runs of short IDs that start in this chunk
  const int64_t cn = min(c + 1, nchunks - 1);  // read only when position p0 + kSegC exists
  const int32_t cs = chunk_start[c], ce = chunk_end[c];
  const int32_t cs2 = chunk_start[cn], ce2 = chunk_end[cn];
  const int64_t pb = (cs == p0 && ce - cs < kSegLong) ? p0 : ce;
  int64_t pe;
  const int64_t q = p0 + kSegC;
  if (q >= N) {
    pe = N;
  } else {
    if (cs2 == q)
      pe = q;
    else if (cs2 < p0)
      pe = pb;  // one run covers the whole chunk: its owner is elsewhere
    else
      pe = (ce2 - cs2 < kSegLong) ? ce2 : cs2;
  }
  pe = min(pe, N);  // [pb, pe) lies in [0, N) already; kept so by the clamps
  if (pe <= pb || pb < 0) return;
  const int64_t col = slice * kSegCols + lane * 4;
  const bool active = col < H;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int64_t colc = active ? col : H - 4;  // a readable column; its results are dropped
  for (int64_t b0 = pb; b0 < pe; b0 += kSegBatch) {
    // every index is clamped into [b0, pe) so that all loads of a batch are
    // issued back to back; entries past pe are masked afterwards (loaded into
    // vector registers: as scalars, the 33 values and 16 row addresses
    // exhaust the scalar registers and the loads serialise)
    int32_t key[kSegBatch + 1], tok[kSegBatch];
#pragma unroll
    for (int i = 0; i <= kSegBatch; ++i) {
      int32_t p = static_cast<int32_t>(min(b0 + i, pe - 1));
      asm volatile("v_mov_b32 %0, %0" : "+v"(p));
      key[i] = skey[p];
      if (i < kSegBatch) tok[i] = sorted[p];
    }
#pragma unroll
    for (int i = 0; i <= kSegBatch; ++i)
      if (b0 + i >= pe) key[i] = -1;  // pe ends a run
    f32x4 row[kSegBatch], cur[kSegBatch];
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) {
      row[i] = load_row4<D>(dout + static_cast<int64_t>(tok[i]) * H, colc);
      cur[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i)
      if (b0 + i >= pe || !active) row[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // dW rows of the runs that end in this batch
    if (accumulate && active) {
#pragma unroll
      for (int i = 0; i < kSegBatch; ++i)
        if (b0 + i < pe && key[i + 1] != key[i])
          cur[i] = *reinterpret_cast<const f32x4*>(dW + static_cast<int64_t>(key[i]) * H + col);
    }
    // sums first (every load of the batch is waited for once), stores after:
    // on this GPU stores count in the same counter as loads, so a store
    // between two uses would make the second wait for the store as well
    bool last[kSegBatch];
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) {
      last[i] = b0 + i < pe && key[i + 1] != key[i];
      if (b0 + i < pe) acc += row[i];
      if (last[i]) {
        row[i] = accumulate ? cur[i] + acc : acc;
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (active) {
#pragma unroll
      for (int i = 0; i < kSegBatch; ++i)
        if (last[i]) *reinterpret_cast<f32x4*>(dW + static_cast<int64_t>(key[i]) * H + col) = row[i];
    }
  }
}

// ------------------------------------------------------------------ candidates

__global__ __launch_bounds__(256) void k_mark(const int32_t* __restrict__ targets, int64_t T,
                                              int64_t V, int32_t* __restrict__ flags) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  const int64_t y = targets[t];
  if (y >= 0 && y < V) flags[y] = 1;
}

__global__ __launch_bounds__(256) void k_emit_unique(const int32_t* __restrict__ flags,
                                                     const int32_t* __restrict__ uidx, int64_t V,
                                                     int32_t* __restrict__ cand) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (v < V && flags[v]) cand[uidx[v]] = static_cast<int32_t>(v);
}

__global__ __launch_bounds__(256) void k_positions(const int32_t* __restrict__ targets, int64_t T,
                                                   int64_t V, const int32_t* __restrict__ uidx,
                                                   int32_t* __restrict__ pos) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  const int64_t y = targets[t];
  pos[t] = (y >= 0 && y < V) ? uidx[y] : static_cast<int32_t>(y);
}

// notin[i] = 1 if perm[i] is a valid row that is not a unique target
__global__ __launch_bounds__(256) void k_notin(const int32_t* __restrict__ perm, int64_t V,
                                               const int32_t* __restrict__ flags,
                                               int32_t* __restrict__ notin) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= V) return;
  const int64_t r = perm[i];
  notin[i] = (r >= 0 && r < V && !flags[r]) ? 1 : 0;
}

__global__ __launch_bounds__(256) void k_emit_neg(const int32_t* __restrict__ perm, int64_t V,
                                                  const int32_t* __restrict__ notin,
                                                  const int32_t* __restrict__ nidx,
                                                  const int32_t* __restrict__ uidx, int64_t P,
                                                  int32_t* __restrict__ cand) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= V || !notin[i]) return;
  const int64_t nu = uidx[V];
  const int64_t need = P > nu ? P - nu : 0;
  const int64_t k = nidx[i];
  if (k < need) cand[nu + k] = perm[i];
}

__global__ void k_cand_counts(const int32_t* __restrict__ uidx, int64_t V, int64_t P,
                              int32_t* n_unique, int32_t* n_cand) {
  if (threadIdx.x == 0) {
    const int32_t nu = uidx[V];
    *n_unique = nu;
    *n_cand = static_cast<int32_t>(P > nu ? P : nu);
  }
}

// One workgroup builds the candidate list for vocabularies up to kCandMaxV
// rows, with the targets' flags as a bit map in LDS: word prefixes of its
// popcounts give every unique target its position; the permutation is read
// in order only as far as the P - |U| negatives it must supply, each ranked
// with wave ballots. Same results as the multi-launch path below (unique
// targets ascending, then the first P - |U| entries of perm that are not
// unique targets).
constexpr int kCandThreads = 1024;
constexpr int kCandLoads = 8;  // global reads in flight per thread
constexpr int64_t kCandMaxV = 262144;

// exclusive prefix of popc(bits[w]) over w < nw into pre[w]; returns the total
__device__ uint32_t cand_word_scan(const uint32_t* bits, uint32_t* pre, int nw, uint32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (nw + kCandThreads - 1) / kCandThreads;
  const int w0 = tid * per;
  uint32_t own = 0;
  for (int k = 0; k < per; ++k)
    if (w0 + k < nw) own += static_cast<uint32_t>(__popc(bits[w0 + k]));
  uint32_t x = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  uint32_t base = 0, total = 0;
  for (int k = 0; k < kCandThreads / 64; ++k) {
    if (k < w) base += wsum[k];
    total += wsum[k];
  }
  uint32_t run = base + x - own;
  for (int k = 0; k < per; ++k)
    if (w0 + k < nw) {
      pre[w0 + k] = run;
      run += static_cast<uint32_t>(__popc(bits[w0 + k]));
    }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kCandThreads) void k_cand_one(const int32_t* __restrict__ targets,
                                                           int64_t T, int64_t V,
                                                           const int32_t* __restrict__ perm,
                                                           int64_t P, int32_t* __restrict__ cand,
                                                           int32_t* __restrict__ pos,
                                                           int32_t* __restrict__ n_unique,
                                                           int32_t* __restrict__ n_cand) {
  constexpr int MAXW = static_cast<int>(kCandMaxV / 32);
  __shared__ uint32_t fbits[MAXW], fpre[MAXW];
  __shared__ uint32_t wsum[kCandThreads / 64];
  __shared__ uint32_t wcnt[2][kCandThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nw = static_cast<int>((V + 31) / 32);
  for (int k = tid; k < nw; k += kCandThreads) fbits[k] = 0u;
  __syncthreads();
  // every global read below is issued kCandLoads at a time: one workgroup
  // has too few waves to hide one round trip per element
  for (int64_t t0 = 0; t0 < T; t0 += kCandThreads * kCandLoads) {
    int32_t y[kCandLoads];
#pragma unroll
    for (int u = 0; u < kCandLoads; ++u) {
      const int64_t t = t0 + u * kCandThreads + tid;
      y[u] = t < T ? targets[t] : -1;
    }
#pragma unroll
    for (int u = 0; u < kCandLoads; ++u)
      if (y[u] >= 0 && y[u] < V) atomicOr(&fbits[y[u] >> 5], 1u << (y[u] & 31));
  }
  __syncthreads();
  const uint32_t nu = cand_word_scan(fbits, fpre, nw, wsum);
  // unique targets, ascending
  for (int k = tid; k < nw; k += kCandThreads) {
    uint32_t b = fbits[k];
    uint32_t at = fpre[k];
    while (b) {
      cand[at++] = k * 32 + (__ffs(b) - 1);
      b &= b - 1u;
    }
  }
  // each target's position among the candidates (other values unchanged)
  for (int64_t t0 = 0; t0 < T; t0 += kCandThreads * kCandLoads) {
    int32_t y[kCandLoads];
#pragma unroll
    for (int u = 0; u < kCandLoads; ++u) {
      const int64_t t = t0 + u * kCandThreads + tid;
      y[u] = t < T ? targets[t] : -1;
    }
#pragma unroll
    for (int u = 0; u < kCandLoads; ++u) {
      const int64_t t = t0 + u * kCandThreads + tid;
      if (t >= T) continue;
      int32_t pt = y[u];
      if (y[u] >= 0 && y[u] < V) {
        const uint32_t b = static_cast<uint32_t>(y[u] & 31);
        pt = static_cast<int32_t>(fpre[y[u] >> 5] + __popc(fbits[y[u] >> 5] & ((1u << b) - 1u)));
      }
      pos[t] = pt;
    }
  }
  // the first P - |U| permutation entries that are valid rows and not
  // targets, in permutation order: read in blocks of kCandThreads * kCandLoads
  // entries (wave w takes kCandLoads groups of 64 in a row), each entry's rank
  // among them = those before its block + those of earlier waves + those of
  // earlier groups and lower lanes of its own wave; reading stops once the
  // ranks reach P - |U|
  const int64_t need = P > nu ? P - nu : 0;
  const uint64_t below = (1ull << lane) - 1ull;
  int64_t found = 0;  // ranks handed out before this block (the same in every thread)
  for (int64_t base = 0, it = 0; base < V && found < need;
       base += kCandThreads * kCandLoads, ++it) {
    int32_t r[kCandLoads];
#pragma unroll
    for (int u = 0; u < kCandLoads; ++u) {
      const int64_t i = base + (static_cast<int64_t>(w) * kCandLoads + u) * 64 + lane;
      r[u] = i < V ? perm[i] : -1;
    }
    uint64_t m[kCandLoads];
    uint32_t cnt = 0;
#pragma unroll
    for (int u = 0; u < kCandLoads; ++u) {
      const bool ni = r[u] >= 0 && r[u] < V && !((fbits[r[u] >> 5] >> (r[u] & 31)) & 1u);
      m[u] = __ballot(ni);
      cnt += static_cast<uint32_t>(__popcll(m[u]));
    }
    // two sets of wave counts, so one barrier per block suffices
    if (lane == 0) wcnt[it & 1][w] = cnt;
    __syncthreads();
    uint32_t wbase = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < kCandThreads / 64; ++k) {
      const uint32_t c = wcnt[it & 1][k];
      if (k < w) wbase += c;
      tot += c;
    }
    int64_t at = found + wbase;
#pragma unroll
    for (int u = 0; u < kCandLoads; ++u) {
      if ((m[u] >> lane) & 1ull) {
        const int64_t q = at + __popcll(m[u] & below);
        if (q < need) cand[nu + q] = r[u];
      }
      at += __popcll(m[u]);
    }
    found += tot;
  }
  if (tid == 0) {
    *n_unique = static_cast<int32_t>(nu);
    *n_cand = static_cast<int32_t>(P > nu ? P : nu);
  }
}

// Gradient scatter of the sampled softmax ([SS] Setup: only the candidate
// rows take part in the loss, so only they receive gradient): candidate row
// i goes to row cand[i] of the table, entries outside [0, V) skipped. The
// candidates are distinct, so this is the scatter-add without the sort: one
// wave per candidate row, kScatLoads float4 per lane in flight. ACC adds into
// the table row; otherwise the row is copied (the launcher zeroes the table
// first). ACC is a template argument: as a run-time branch inside the row
// loop it doubled the kernel's time.
constexpr int kScatLoads = 8;
template <bool ACC>
__global__ __launch_bounds__(256) void k_scatter_rows(const int32_t* __restrict__ cand, int64_t P,
                                                      const float* __restrict__ src, int64_t H,
                                                      int64_t V, float* __restrict__ dW) {
  const int lane = threadIdx.x & 63;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (i >= P) return;
  const int64_t v = cand[i];
  if (v < 0 || v >= V) return;
  const f32x4* s = reinterpret_cast<const f32x4*>(src + i * H);
  f32x4* d = reinterpret_cast<f32x4*>(dW + v * H);
  const int64_t n4 = H / 4;
  for (int64_t j0 = 0; j0 < n4; j0 += 64 * kScatLoads) {
    f32x4 x[kScatLoads], y[kScatLoads];
#pragma unroll
    for (int u = 0; u < kScatLoads; ++u) {
      const int64_t j = j0 + u * 64 + lane;
      if (j < n4) {
        x[u] = s[j];
        if constexpr (ACC) y[u] = d[j];
      }
    }
#pragma unroll
    for (int u = 0; u < kScatLoads; ++u) {
      const int64_t j = j0 + u * 64 + lane;
      if (j < n4) {
        if constexpr (ACC)
          d[j] = y[u] + x[u];
        else
          d[j] = x[u];
      }
    }
  }
}

// dW[rows[i]] = 0 for rows[i] in [0, V): one wave per row, 8 float4 stores
// per lane in flight.
__global__ __launch_bounds__(256) void k_zero_rows(const int32_t* __restrict__ rows, int64_t n,
                                                   int64_t H, int64_t V, float* __restrict__ dW) {
  const int lane = threadIdx.x & 63;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (i >= n) return;
  const int64_t v = rows[i];
  if (v < 0 || v >= V) return;
  f32x4* d = reinterpret_cast<f32x4*>(dW + v * H);
  const int64_t n4 = H / 4;
  for (int64_t j = lane; j < n4; j += 64) d[j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ------------------------------------------------------------------ launchers

hipError_t run_emb_fwd(const int32_t* ids, const void* W, int64_t T, int64_t H, int64_t V_real,
                       const SegTable& sg, size_t esize, void* out, int32_t* n_bad,
                       hipStream_t s) {
  if (T == 0) {
    if (!n_bad) return hipSuccess;
    hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(64), 0, s, n_bad);
    return hipGetLastError();
  }
  const int64_t row_bytes = H * static_cast<int64_t>(esize);
  const int64_t blocks = cdiv(T, 4 * kRowsPerWave);
  hipLaunchKernelGGL(k_vemb_fwd, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, ids,
                     static_cast<const char*>(W), T, row_bytes, V_real, sg,
                     static_cast<char*>(out), n_bad);
  return hipGetLastError();
}

hipError_t run_emb_bwd(const int32_t* ids, const void* dout, bool dout_bf16, int64_t T, int64_t H,
                       int64_t V_real, int64_t V_pad, float* dW, int32_t accumulate,
                       const EmbBwdPlan& p, hipStream_t s) {
  hipError_t err;
  if (!accumulate) {
    const int64_t n4 = V_pad * H / 4;
    hipLaunchKernelGGL(k_fill_f4, dim3(static_cast<uint32_t>(cdiv(n4, 256))), dim3(256), 0, s,
                       reinterpret_cast<float4*>(dW), n4);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (T == 0) return hipSuccess;
  // 1. stable sort of the tokens by ID
  if (p.runs) {
    hipLaunchKernelGGL(k_run_sort, dim3(static_cast<uint32_t>(p.nruns)), dim3(kRun), 0, s, ids, T,
                       V_real, p.vbits, p.rid, p.rtok, p.rvalid, p.n_long);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(k_run_merge, dim3(static_cast<uint32_t>(p.nruns * kMergeSplit)),
                       dim3(4 * kRankTok), 0, s, p.rid,
                       p.rtok, p.rvalid, static_cast<int32_t>(p.nruns), p.sorted, p.skey,
                       p.n_sorted, p.chunk_start, p.chunk_end, p.long_runs, p.n_long,
                       static_cast<int32_t>(p.nchunks));
    if ((err = hipGetLastError()) != hipSuccess) return err;
  } else {
    const int64_t ncnt = p.nblocks * V_real;
    if (ncnt % 4 == 0) {
      hipLaunchKernelGGL(k_fill_i32x4, dim3(static_cast<uint32_t>(cdiv(ncnt / 4, 256))),
                         dim3(256), 0, s, reinterpret_cast<int4*>(p.bcnt), ncnt / 4);
    } else {
      hipLaunchKernelGGL(k_fill_i32, dim3(static_cast<uint32_t>(cdiv(ncnt, kScanThreads))),
                         dim3(kScanThreads), 0, s, p.bcnt, ncnt, 0);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(k_block_sort, dim3(static_cast<uint32_t>(p.nblocks)), dim3(kSortThreads), 0,
                       s, ids, T, V_real, p.lkey, p.lrank, p.bcnt, p.n_long);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(k_col_scan, dim3(static_cast<uint32_t>(cdiv(V_real, 256))), dim3(256), 0, s,
                       p.bcnt, p.nblocks, V_real, p.counts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = run_scan(p.counts, V_real, p.offs, nullptr, p.scan_tmp, s)) != hipSuccess)
      return err;
    const int64_t nkeys = p.nblocks * kSortBlock;
    hipLaunchKernelGGL(k_place_sorted, dim3(static_cast<uint32_t>(cdiv(nkeys, 256))), dim3(256), 0,
                       s, p.lkey, p.lrank, p.bcnt, p.offs, nkeys, V_real, p.sorted, p.skey);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(k_chunk_starts, dim3(static_cast<uint32_t>(cdiv(p.nchunks, 256))),
                       dim3(256), 0, s, p.skey, p.offs, p.n_sorted, p.nchunks, p.chunk_start,
                       p.chunk_end, p.long_runs, p.n_long);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // 2. segment sums: long IDs by column slices, the others by chunks
  const int64_t nwg = p.long_wgs + p.nchunks * cdiv(p.nslices, 4);
  const dim3 grid(static_cast<uint32_t>(nwg));
  if (dout_bf16)
    hipLaunchKernelGGL(k_seg_sums<uint16_t>, grid, dim3(256), 0, s, p.skey, p.sorted, p.n_sorted,
                       p.chunk_start, p.chunk_end, p.long_runs, p.n_long,
                       static_cast<const uint16_t*>(dout), H, p.nslices, p.nchunks, p.long_wgs,
                       dW, accumulate);
  else
    hipLaunchKernelGGL(k_seg_sums<float>, grid, dim3(256), 0, s, p.skey, p.sorted, p.n_sorted,
                       p.chunk_start, p.chunk_end, p.long_runs, p.n_long,
                       static_cast<const float*>(dout), H, p.nslices, p.nchunks, p.long_wgs, dW,
                       accumulate);
  return hipGetLastError();
}

// The candidate rows' copy (add = false) or add into dW, no fill.
static hipError_t scatter_rows(const int32_t* cand, int64_t P, const float* dWc, int64_t H,
                               int64_t V, float* dW, bool add, hipStream_t s) {
  if (P == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>(cdiv(P, 4)));
  if (add)
    hipLaunchKernelGGL(k_scatter_rows<true>, grid, dim3(256), 0, s, cand, P, dWc, H, V, dW);
  else
    hipLaunchKernelGGL(k_scatter_rows<false>, grid, dim3(256), 0, s, cand, P, dWc, H, V, dW);
  return hipGetLastError();
}

hipError_t run_ss_scatter(const int32_t* cand, int64_t P, const float* dWc, int64_t H, int64_t V,
                          float* dW, int32_t accumulate, hipStream_t s) {
  if (!accumulate) {
    const int64_t n4 = V * H / 4;
    hipLaunchKernelGGL(k_fill_f4, dim3(static_cast<uint32_t>(cdiv(n4, 256))), dim3(256), 0, s,
                       reinterpret_cast<float4*>(dW), n4);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return scatter_rows(cand, P, dWc, H, V, dW, accumulate != 0, s);
}

hipError_t run_ss_scatter_replace(const int32_t* prev, int64_t P_prev, const int32_t* cand,
                                  int64_t P, const float* dWc, int64_t H, int64_t V, float* dW,
                                  hipStream_t s) {
  if (P_prev > 0) {
    hipLaunchKernelGGL(k_zero_rows, dim3(static_cast<uint32_t>(cdiv(P_prev, 4))), dim3(256), 0, s,
                       prev, P_prev, H, V, dW);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return scatter_rows(cand, P, dWc, H, V, dW, false, s);  // rows of a zero table: copy
}

hipError_t run_candidates(const int32_t* targets, int64_t T, int64_t V, const int32_t* perm,
                          int64_t P, int32_t* cand, int32_t* pos, int32_t* n_unique,
                          int32_t* n_cand, const CandPlan& p, hipStream_t s) {
  hipError_t err;
  if (V <= kCandMaxV) {
    hipLaunchKernelGGL(k_cand_one, dim3(1), dim3(kCandThreads), 0, s, targets, T, V, perm, P,
                       cand, pos, n_unique, n_cand);
    return hipGetLastError();
  }
  const uint32_t vb = static_cast<uint32_t>(cdiv(V, 256));
  hipLaunchKernelGGL(k_fill_i32, dim3(static_cast<uint32_t>(cdiv(V, kScanThreads))),
                     dim3(kScanThreads), 0, s, p.flags, V, 0);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (T > 0) {
    hipLaunchKernelGGL(k_mark, dim3(static_cast<uint32_t>(cdiv(T, 256))), dim3(256), 0, s, targets,
                       T, V, p.flags);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if ((err = run_scan(p.flags, V, p.uidx, nullptr, p.scan_tmp, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(k_emit_unique, dim3(vb), dim3(256), 0, s, p.flags, p.uidx, V, cand);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (T > 0) {
    hipLaunchKernelGGL(k_positions, dim3(static_cast<uint32_t>(cdiv(T, 256))), dim3(256), 0, s,
                       targets, T, V, p.uidx, pos);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_notin, dim3(vb), dim3(256), 0, s, perm, V, p.flags, p.notin);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = run_scan(p.notin, V, p.nidx, nullptr, p.scan_tmp, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(k_emit_neg, dim3(vb), dim3(256), 0, s, perm, V, p.notin, p.nidx, p.uidx, P,
                     cand);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_cand_counts, dim3(1), dim3(64), 0, s, p.uidx, V, P, n_unique, n_cand);
  return hipGetLastError();
}

}  // namespace vce
