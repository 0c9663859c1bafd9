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
// Deterministic, one writer per row:
//   count IDs -> exclusive scan -> group token indices by ID -> order each
//   group by token index -> segment sums in fixed-size chunks of the sorted
//   list (balanced even under Zipf skew) -> a fix-up that adds, in order,
//   the partial sums of groups that span chunks.
#include "vce_device.hpp"
#include "vce_internal.hpp"

namespace vce {

constexpr int kScanThreads = 256;
constexpr int kScanPerThread = 16;
constexpr int kScanBlock = kScanThreads * kScanPerThread;  // 4096 values per block
constexpr int kSegChunk = 16;                              // sorted positions per chunk
constexpr int kSegCols = 256;                              // dW columns per wave (64 lanes x 4)

// ------------------------------------------------------------------ planning

int64_t scan_blocks(int64_t n) { return cdiv(n < 1 ? 1 : n, kScanBlock); }

EmbBwdPlan plan_emb_bwd(int64_t T, int64_t H, int64_t V_real, void* ws) {
  EmbBwdPlan p{};
  p.nchunks = cdiv(T < 1 ? 1 : T, kSegChunk);
  p.nslices = cdiv(H, kSegCols);
  p.scan_blocks = scan_blocks(V_real);
  Carve c(ws);
  p.counts = c.take<int32_t>(static_cast<size_t>(V_real));
  p.offs = c.take<int32_t>(static_cast<size_t>(V_real + 1));
  p.cursor = c.take<int32_t>(static_cast<size_t>(V_real + 1));
  p.perm = c.take<int32_t>(static_cast<size_t>(T < 1 ? 1 : T));
  p.sorted = c.take<int32_t>(static_cast<size_t>(T < 1 ? 1 : T));
  p.scan_tmp = c.take<int32_t>(static_cast<size_t>(p.scan_blocks + 1));
  p.partial = c.take<float>(static_cast<size_t>(p.nchunks * 2 * H));
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

// One wave per output row; 16-byte pieces. bytes_per_row is a multiple of 16.
__global__ __launch_bounds__(256) void k_vemb_fwd(const int32_t* __restrict__ ids,
                                                  const char* __restrict__ W, int64_t T,
                                                  int64_t row_bytes, int64_t V_real, int64_t S,
                                                  char* __restrict__ out, int32_t* n_bad) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t id = ids[t];
  const int64_t nvec = row_bytes >> 4;
  u32x4* dst = reinterpret_cast<u32x4*>(out + t * row_bytes);
  // owner test, then the local index within the owner's slice
  const bool owned = (id >= 0) && (id < V_real);
  if (owned) {
    const int64_t k = id / S;
    const int64_t local = id - k * S;
    const u32x4* src = reinterpret_cast<const u32x4*>(W + (k * S + local) * row_bytes);
    int64_t c = lane;
    for (; c + 192 < nvec; c += 256) {
      // table rows are read through the caches: repeated IDs hit them again
      const u32x4 a = src[c];
      const u32x4 b = src[c + 64];
      const u32x4 d = src[c + 128];
      const u32x4 e = src[c + 192];
      __builtin_nontemporal_store(a, dst + c);
      __builtin_nontemporal_store(b, dst + c + 64);
      __builtin_nontemporal_store(d, dst + c + 128);
      __builtin_nontemporal_store(e, dst + c + 192);
    }
    for (; c < nvec; c += 64) __builtin_nontemporal_store(src[c], dst + c);
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t c = lane; c < nvec; c += 64) __builtin_nontemporal_store(z, dst + c);
    if (lane == 0 && n_bad) atomicAdd(n_bad, 1);
  }
}

__global__ void k_zero_i32(int32_t* p) {
  if (threadIdx.x == 0) *p = 0;
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

__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ ids, int64_t T,
                                              int64_t V_real, int32_t* __restrict__ counts) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  const int64_t id = ids[t];
  if (id >= 0 && id < V_real) atomicAdd(counts + id, 1);
}

// token indices grouped by ID (order inside a group is arbitrary here)
__global__ __launch_bounds__(256) void k_place(const int32_t* __restrict__ ids, int64_t T,
                                               int64_t V_real, int32_t* __restrict__ cursor,
                                               int32_t* __restrict__ perm) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  const int64_t id = ids[t];
  if (id >= 0 && id < V_real) perm[atomicAdd(cursor + id, 1)] = static_cast<int32_t>(t);
}

// sorted[a + rank] = t, where rank = number of tokens of the same ID smaller than t
__global__ __launch_bounds__(256) void k_rank(const int32_t* __restrict__ ids,
                                              const int32_t* __restrict__ perm,
                                              const int32_t* __restrict__ offs,
                                              const int32_t* __restrict__ counts, int64_t T,
                                              int64_t V_real, int32_t* __restrict__ sorted) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t N = offs[V_real];
  if (p >= N || p >= T) return;
  const int32_t t = perm[p];
  const int64_t id = ids[t];
  const int64_t a = offs[id];
  const int64_t len = counts[id];
  int64_t rank = 0;
  for (int64_t q = a; q < a + len; ++q) rank += (perm[q] < t) ? 1 : 0;
  sorted[a + rank] = t;
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

// One wave per (chunk of kSegChunk sorted positions, 256-column slice).
// Runs of one ID that lie wholly in the chunk are added into dW here; runs
// that continue into a neighbouring chunk leave a partial sum: slot 0 for
// the run that began in an earlier chunk, slot 1 for the run that begins
// here and continues.
template <typename D>
__global__ __launch_bounds__(256) void k_segsum(const int32_t* __restrict__ ids,
                                                const int32_t* __restrict__ sorted,
                                                const int32_t* __restrict__ offs,
                                                const int32_t* __restrict__ counts,
                                                const D* __restrict__ dout, int64_t T, int64_t H,
                                                int64_t V_real, int64_t nslices,
                                                float* __restrict__ dW, int32_t accumulate,
                                                float* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int64_t slice = static_cast<int64_t>(blockIdx.y) * 4 + (threadIdx.x >> 6);
  const int64_t c = blockIdx.x;
  const int64_t N = offs[V_real];
  const int64_t p0 = c * kSegChunk;
  if (slice >= nslices || p0 >= N) return;
  const int64_t p1 = min(p0 + kSegChunk, N);
  const int64_t col = slice * kSegCols + lane * 4;
  const bool active = col < H;
  int32_t tk[kSegChunk];
  int32_t key[kSegChunk];
  f32x4 row[kSegChunk];
#pragma unroll
  for (int i = 0; i < kSegChunk; ++i) {
    const bool in = p0 + i < p1;
    tk[i] = in ? sorted[p0 + i] : 0;
    key[i] = in ? ids[tk[i]] : -1;
  }
#pragma unroll
  for (int i = 0; i < kSegChunk; ++i) {
    if (p0 + i < p1 && active)
      row[i] = load_row4<D>(dout + static_cast<int64_t>(tk[i]) * H, col);
    else
      row[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kSegChunk; ++i) {
    if (p0 + i >= p1) break;
    acc += row[i];
    const bool last = (p0 + i + 1 == p1) || (key[i + (i + 1 < kSegChunk ? 1 : 0)] != key[i]) ||
                      (i + 1 == kSegChunk);
    if (last) {
      const int64_t v = key[i];
      const int64_t a = offs[v];
      const int64_t b = a + counts[v];
      if (active) {
        if (a >= p0 && b <= p1) {
          f32x4* dst = reinterpret_cast<f32x4*>(dW + v * H + col);
          if (accumulate) {
            f32x4 cur = *dst;
            cur += acc;
            *dst = cur;
          } else {
            *dst = acc;
          }
        } else {
          const int slot = (a < p0) ? 0 : 1;
          *reinterpret_cast<f32x4*>(partial + (c * 2 + slot) * H + col) = acc;
        }
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// A group that begins in chunk c and continues past it: add slot 1 of c and
// slot 0 of each following chunk it covers, in chunk order.
__global__ __launch_bounds__(256) void k_segfix(const int32_t* __restrict__ ids,
                                                const int32_t* __restrict__ sorted,
                                                const int32_t* __restrict__ offs,
                                                const int32_t* __restrict__ counts, int64_t H,
                                                int64_t V_real, int64_t nslices,
                                                float* __restrict__ dW, int32_t accumulate,
                                                const float* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int64_t slice = static_cast<int64_t>(blockIdx.y) * 4 + (threadIdx.x >> 6);
  const int64_t c = blockIdx.x;
  const int64_t N = offs[V_real];
  const int64_t p0 = c * kSegChunk;
  if (slice >= nslices || p0 >= N) return;
  const int64_t p1 = min(p0 + kSegChunk, N);
  const int64_t v = ids[sorted[p1 - 1]];
  const int64_t a = offs[v];
  const int64_t b = a + counts[v];
  if (!(a >= p0 && b > p1)) return;
  const int64_t col = slice * kSegCols + lane * 4;
  if (col >= H) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(partial + (c * 2 + 1) * H + col);
  const int64_t last = (b - 1) / kSegChunk;
  for (int64_t cc = c + 1; cc <= last; ++cc)
    acc += *reinterpret_cast<const f32x4*>(partial + (cc * 2 + 0) * H + col);
  f32x4* dst = reinterpret_cast<f32x4*>(dW + v * H + col);
  if (accumulate) {
    f32x4 cur = *dst;
    cur += acc;
    *dst = cur;
  } else {
    *dst = acc;
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

// ------------------------------------------------------------------ launchers

hipError_t run_emb_fwd(const int32_t* ids, const void* W, int64_t T, int64_t H, int64_t V_real,
                       int64_t V_pad, int32_t n, size_t esize, void* out, int32_t* n_bad,
                       hipStream_t s) {
  hipError_t err;
  if (n_bad) {
    hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(64), 0, s, n_bad);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (T == 0) return hipSuccess;
  const int64_t S = V_pad / n;
  hipLaunchKernelGGL(k_vemb_fwd, dim3(static_cast<uint32_t>(cdiv(T, 4))), dim3(256), 0, s, ids,
                     static_cast<const char*>(W), T, H * static_cast<int64_t>(esize), V_real, S,
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
  const uint32_t tb = static_cast<uint32_t>(cdiv(T, 256));
  hipLaunchKernelGGL(k_fill_i32, dim3(static_cast<uint32_t>(cdiv(V_real, kScanThreads))),
                     dim3(kScanThreads), 0, s, p.counts, V_real, 0);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_hist, dim3(tb), dim3(256), 0, s, ids, T, V_real, p.counts);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = run_scan(p.counts, V_real, p.offs, p.cursor, p.scan_tmp, s)) != hipSuccess) return err;
  hipLaunchKernelGGL(k_place, dim3(tb), dim3(256), 0, s, ids, T, V_real, p.cursor, p.perm);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_rank, dim3(tb), dim3(256), 0, s, ids, p.perm, p.offs, p.counts, T, V_real,
                     p.sorted);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const dim3 grid(static_cast<uint32_t>(p.nchunks), static_cast<uint32_t>(cdiv(p.nslices, 4)));
  if (dout_bf16)
    hipLaunchKernelGGL(k_segsum<uint16_t>, grid, dim3(256), 0, s, ids, p.sorted, p.offs, p.counts,
                       static_cast<const uint16_t*>(dout), T, H, V_real, p.nslices, dW,
                       accumulate, p.partial);
  else
    hipLaunchKernelGGL(k_segsum<float>, grid, dim3(256), 0, s, ids, p.sorted, p.offs, p.counts,
                       static_cast<const float*>(dout), T, H, V_real, p.nslices, dW, accumulate,
                       p.partial);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_segfix, grid, dim3(256), 0, s, ids, p.sorted, p.offs, p.counts, H, V_real,
                     p.nslices, dW, accumulate, p.partial);
  return hipGetLastError();
}

hipError_t run_candidates(const int32_t* targets, int64_t T, int64_t V, const int32_t* perm,
                          int64_t P, int32_t* cand, int32_t* pos, int32_t* n_unique,
                          int32_t* n_cand, const CandPlan& p, hipStream_t s) {
  hipError_t err;
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
