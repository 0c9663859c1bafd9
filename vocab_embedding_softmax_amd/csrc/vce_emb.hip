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
// Deterministic, one writer per row, no atomics:
//   per block of 1024 tokens, an LDS sort by (ID, token) with per-block ID
//   counts -> per-ID offsets over the blocks -> exclusive scan over IDs ->
//   stable placement of every token -> segment sums in fixed-size chunks of
//   the sorted list (balanced even under Zipf skew) -> a fix-up that adds the
//   partial sums of groups that span chunks in a fixed order.
#include "vce_device.hpp"
#include "vce_internal.hpp"

namespace vce {

constexpr int kScanThreads = 256;
constexpr int kScanPerThread = 16;
constexpr int kScanBlock = kScanThreads * kScanPerThread;  // 4096 values per block
constexpr int kSegChunk = 16;                              // sorted positions per chunk
constexpr int kSegBatch = 16;                              // rows loaded together
constexpr int kSegCols = 256;                              // dW columns per wave (64 lanes x 4)
constexpr int kSortBlock = 1024;                           // tokens per local sort
constexpr int kSortThreads = 512;

// ------------------------------------------------------------------ planning

int64_t scan_blocks(int64_t n) { return cdiv(n < 1 ? 1 : n, kScanBlock); }

EmbBwdPlan plan_emb_bwd(int64_t T, int64_t H, int64_t V_real, void* ws) {
  EmbBwdPlan p{};
  const int64_t Tp = T < 1 ? 1 : T;
  p.nblocks = cdiv(Tp, kSortBlock);
  p.nchunks = cdiv(Tp, kSegChunk);
  p.nslices = cdiv(H, kSegCols);
  p.scan_blocks = scan_blocks(V_real);
  Carve c(ws);
  p.bcnt = c.take<int32_t>(static_cast<size_t>(p.nblocks * V_real));
  p.counts = c.take<int32_t>(static_cast<size_t>(V_real));
  p.offs = c.take<int32_t>(static_cast<size_t>(V_real + 1));
  p.lkey = c.take<uint64_t>(static_cast<size_t>(p.nblocks * kSortBlock));
  p.lrank = c.take<int32_t>(static_cast<size_t>(p.nblocks * kSortBlock));
  p.sorted = c.take<int32_t>(static_cast<size_t>(Tp));
  p.skey = c.take<int32_t>(static_cast<size_t>(Tp));
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

// One wave per output row, in 16-byte pieces: every load of the row is in
// flight before the first store. row_bytes is a multiple of 16.
__global__ __launch_bounds__(256) void k_vemb_fwd(const int32_t* __restrict__ ids,
                                                  const char* __restrict__ W, int64_t T,
                                                  int64_t row_bytes, int64_t V_real, int64_t S,
                                                  char* __restrict__ out, int32_t* n_bad) {
  constexpr int U = 8;  // pieces per lane held at once
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t id = ids[t];
  const int64_t nvec = row_bytes >> 4;
  u32x4* dst = reinterpret_cast<u32x4*>(out + t * row_bytes);
  // owner test, then the local index within the owner's slice
  const bool owned = (id >= 0) && (id < V_real);
  if (!owned && lane == 0 && n_bad) atomicAdd(n_bad, 1);
  const u32x4* src = nullptr;
  if (owned) {
    const int64_t k = id / S;
    const int64_t local = id - k * S;
    src = reinterpret_cast<const u32x4*>(W + (k * S + local) * row_bytes);
  }
  for (int64_t c0 = 0; c0 < nvec; c0 += 64 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + lane + 64 * u;
      v[u] = (owned && c < nvec) ? src[c] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + lane + 64 * u;
      if (c < nvec) __builtin_nontemporal_store(v[u], dst + c);
    }
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
                                                             int32_t* __restrict__ bcnt) {
  __shared__ uint64_t s[kSortBlock];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
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

// One wave per (chunk of kSegChunk sorted positions, 256-column slice).
// Runs of one ID that lie wholly in the chunk are added into dW here; runs
// that continue into a neighbouring chunk leave a partial sum: slot 0 for
// the run that began in an earlier chunk, slot 1 for the run that begins
// here and continues. Rows are summed in sorted (= increasing token) order.
template <typename D>
__global__ __launch_bounds__(256) void k_segsum(const int32_t* __restrict__ skey,
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
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int32_t next_key = skey[p0];
  for (int64_t b0 = p0; b0 < p1; b0 += kSegBatch) {
    int32_t key[kSegBatch + 1];
    f32x4 row[kSegBatch];
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) {
      const int64_t p = b0 + i;
      int32_t tk = 0;
      if (p < p1) tk = sorted[p];
      key[i] = (i == 0) ? next_key : ((p < p1) ? skey[p] : -1);
      if (p < p1 && active)
        row[i] = load_row4<D>(dout + static_cast<int64_t>(tk) * H, col);
      else
        row[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    {
      const int64_t p = b0 + kSegBatch;
      key[kSegBatch] = (p < p1) ? skey[p] : -1;
      next_key = key[kSegBatch];
    }
#pragma unroll
    for (int i = 0; i < kSegBatch; ++i) {
      const int64_t p = b0 + i;
      if (p >= p1) break;
      acc += row[i];
      if (p + 1 == p1 || key[i + 1] != key[i]) {  // last position of a run
        const int64_t v = key[i];
        const int64_t a = offs[v];
        const int64_t e = a + counts[v];
        if (active) {
          if (a >= p0 && e <= p1) {
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
}

// A group that begins in chunk c and continues past it: slot 1 of c plus
// slot 0 of every following chunk it covers, added in a fixed pattern
// (eight interleaved partial sums, then combined in a fixed tree).
__global__ __launch_bounds__(256) void k_segfix(const int32_t* __restrict__ skey,
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
  const int64_t v = skey[p1 - 1];
  const int64_t a = offs[v];
  const int64_t e = a + counts[v];
  if (!(a >= p0 && e > p1)) return;
  const int64_t col = slice * kSegCols + lane * 4;
  if (col >= H) return;
  const int64_t last = (e - 1) / kSegChunk;
  f32x4 part[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) part[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t cc = c + 1; cc <= last; cc += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (cc + u <= last)
        part[u] += *reinterpret_cast<const f32x4*>(partial + ((cc + u) * 2 + 0) * H + col);
  }
  f32x4 acc = *reinterpret_cast<const f32x4*>(partial + (c * 2 + 1) * H + col);
  acc += ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
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
  // 1. stable sort of the tokens by ID
  const int64_t ncnt = p.nblocks * V_real;
  if (ncnt % 4 == 0) {
    hipLaunchKernelGGL(k_fill_i32x4, dim3(static_cast<uint32_t>(cdiv(ncnt / 4, 256))), dim3(256),
                       0, s, reinterpret_cast<int4*>(p.bcnt), ncnt / 4);
  } else {
    hipLaunchKernelGGL(k_fill_i32, dim3(static_cast<uint32_t>(cdiv(ncnt, kScanThreads))),
                       dim3(kScanThreads), 0, s, p.bcnt, ncnt, 0);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_block_sort, dim3(static_cast<uint32_t>(p.nblocks)), dim3(kSortThreads), 0, s,
                     ids, T, V_real, p.lkey, p.lrank, p.bcnt);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_col_scan, dim3(static_cast<uint32_t>(cdiv(V_real, 256))), dim3(256), 0, s,
                     p.bcnt, p.nblocks, V_real, p.counts);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = run_scan(p.counts, V_real, p.offs, nullptr, p.scan_tmp, s)) != hipSuccess) return err;
  const int64_t nkeys = p.nblocks * kSortBlock;
  hipLaunchKernelGGL(k_place_sorted, dim3(static_cast<uint32_t>(cdiv(nkeys, 256))), dim3(256), 0, s,
                     p.lkey, p.lrank, p.bcnt, p.offs, nkeys, V_real, p.sorted, p.skey);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // 2. segment sums in fixed-size chunks of the sorted list, then the fix-up
  const dim3 grid(static_cast<uint32_t>(p.nchunks), static_cast<uint32_t>(cdiv(p.nslices, 4)));
  if (dout_bf16)
    hipLaunchKernelGGL(k_segsum<uint16_t>, grid, dim3(256), 0, s, p.skey, p.sorted, p.offs, p.counts,
                       static_cast<const uint16_t*>(dout), T, H, V_real, p.nslices, dW,
                       accumulate, p.partial);
  else
    hipLaunchKernelGGL(k_segsum<float>, grid, dim3(256), 0, s, p.skey, p.sorted, p.offs, p.counts,
                       static_cast<const float*>(dout), T, H, V_real, p.nslices, dW, accumulate,
                       p.partial);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_segfix, grid, dim3(256), 0, s, p.skey, p.offs, p.counts, H, V_real,
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
