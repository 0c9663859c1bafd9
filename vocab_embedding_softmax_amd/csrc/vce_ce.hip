// Cross-entropy forward and backward over a vocabulary-sharded LM head.
//
// Forward ("Vocabulary shards: look up locally and normalize globally", ¶3-4):
//   1. k_gemm_tn<EPI_FWD>: every vocabulary tile of every shard computes its
//      logits h W_tile^T with MFMA and reduces them at once to per-token
//      (max, sum exp) over its real rows; the tile that owns a token's target
//      stores that logit. Logits never leave registers.
//   2. k_ce_merge: per token, the tiles of each shard are merged into the
//      shard's (m_k, s_k) (the quantities one rank would hold), then the
//      shards are merged into the global log-sum-exp, in a fixed order.
//   3. k_ce_finalize: fixed-order sum of the loss and the token counts.
// Backward (same page, ¶4), one vocabulary chunk at a time (a shard, or a
//   piece of one): logits of the chunk are recomputed tile by tile to form
//   G = scale * (softmax - onehot) for the chunk's columns, staged token-major
//   in the input type ([T][chunk], never [T][V]); then dh += G W_chunk (the
//   partial a vocabulary rank would contribute to the all-reduce) and
//   dW_chunk = G^T h, both MFMA GEMMs that read G, W and h in place (the
//   K-major operands through transposing LDS reads).
#include <mutex>

#include "gemm_tn.hpp"
#include "vce_internal.hpp"

namespace vce {

// ------------------------------------------------------------ static scratch

// Device memory of the allocation-free argmax (the per-tile reports that
// vce_argmax keeps in the caller's workspace). Each GPU the library runs on
// holds its own copy until the process ends. In host code `scratch` is only a
// host-side stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------------ planning

SegTable shard_segments(int32_t n, const int64_t* rows, int64_t V_pad) {
  SegTable sg{};
  sg.n = n;
  int32_t tiles = 0;
  for (int32_t k = 0; k <= n; ++k) {
    sg.row[k] = rows ? rows[k] : (V_pad / n) * k;
    sg.tile[k] = tiles;
    if (k < n) {
      const int64_t len = (rows ? rows[k + 1] : (V_pad / n) * (k + 1)) - sg.row[k];
      tiles += static_cast<int32_t>(cdiv(len, kTileM));
    }
  }
  return sg;
}

SegTable one_segment(int64_t rows) {
  SegTable sg{};
  sg.n = 1;
  sg.row[0] = 0;
  sg.row[1] = rows;
  sg.tile[0] = 0;
  sg.tile[1] = static_cast<int32_t>(cdiv(rows, kTileM));
  return sg;
}

FwdPlan plan_fwd(int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t n,
                 const int64_t* rows, void* ws) {
  (void)H;
  (void)V_real;
  FwdPlan p{};
  p.seg = shard_segments(n, rows, V_pad);
  p.tiles_m = p.seg.tile[n];
  p.tiles_n = cdiv(T, kTileN);
  p.merge_blocks = cdiv(T, kMergeTok);
  Carve c(ws);
  p.stats = c.take<float2>(static_cast<size_t>(p.tiles_m * T));
  p.zt = c.take<float>(static_cast<size_t>(T));
  p.part_loss = c.take<float>(static_cast<size_t>(p.merge_blocks + 1));
  p.part_nv = c.take<int32_t>(static_cast<size_t>(p.merge_blocks + 1));
  p.part_nb = c.take<int32_t>(static_cast<size_t>(p.merge_blocks + 1));
  p.bytes = c.used;
  return p;
}

ArgPlan plan_argmax(int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t n,
                    const int64_t* rows, void* ws) {
  (void)H;
  (void)V_real;
  ArgPlan p{};
  p.seg = shard_segments(n, rows, V_pad);
  p.tiles_m = p.seg.tile[n];
  p.tiles_n = cdiv(T, kTileN);
  Carve c(ws);
  p.val = c.take<float>(static_cast<size_t>(p.tiles_m * T));
  p.idx = c.take<int32_t>(static_cast<size_t>(p.tiles_m * T));
  p.bytes = c.used;
  return p;
}

int32_t k_splits_for(int64_t tiles, int64_t K, int64_t out_elems) {
  constexpr int64_t kCUs = 256;
  constexpr int32_t kMaxSplit = 8;
  if (tiles <= 0) return 1;
  // Estimated time in units of one 64-K slice of one tile on one CU
  // (≈ 1.65 µs at the GEMMs' rate): rounds of tiles over the CUs, each tile
  // its share of K plus ≈ 4 slices of fixed cost (prologue, epilogue); a
  // split also writes s - 1 float32 planes and a pass reads them and the
  // output and writes the output (≈ 5 TB/s, i.e. ≈ 8.25 MB per slice time).
  auto cost = [&](int64_t s) {
    const double rounds = static_cast<double>(cdiv(tiles * s, kCUs));
    const double gemm = rounds * static_cast<double>(cdiv(K, s * 64) + 4);
    if (s == 1) return gemm;
    const double bytes = static_cast<double>(out_elems) * 4.0 * static_cast<double>(2 * (s - 1) + 2);
    return gemm + bytes / 8.25e6 + 3.0;
  };
  int32_t best = 1;
  double best_cost = cost(1);
  for (int32_t s = 2; s <= kMaxSplit; ++s) {
    if (cdiv(K, s) < 1024) break;
    const double c = cost(s);
    if (c < best_cost * 0.98) {  // a split must save at least 2 %
      best = s;
      best_cost = c;
    }
  }
  return best;
}

TailSplit tail_split_for(int64_t rows, int64_t tiles_n, int64_t K, int64_t n_cols) {
  constexpr int64_t kCUs = 256;
  const int64_t tiles_m = cdiv(rows, kTileM);
  TailSplit best{rows, 1};
  if (tiles_m <= 0 || tiles_n <= 0 || (tiles_m * tiles_n) % kCUs == 0) return best;
  // the most whole rows of tiles that fit in the whole rounds
  const int64_t m1 = (tiles_m * tiles_n / kCUs) * kCUs / tiles_n;
  if (m1 == 0 || m1 == tiles_m) return best;
  const int64_t rest = (tiles_m - m1) * tiles_n;  // tiles left for the last round
  // as many parts as fill one round, each at least 1024 K positions
  const int32_t ks = static_cast<int32_t>(min(kCUs / rest, max(K / 1024, int64_t{1})));
  if (ks < 2) return best;
  // units of one 64-K slice of one tile, as in k_splits_for
  const double slices = static_cast<double>(cdiv(K, 64));
  const double whole = static_cast<double>(cdiv(tiles_m * tiles_n, kCUs)) * (slices + 4.0);
  const double tail_rows = static_cast<double>(rows - m1 * kTileM);
  const double split = static_cast<double>(cdiv(m1 * tiles_n, kCUs)) * (slices + 4.0) +
                       static_cast<double>(cdiv(K, ks * 64) + 4) +
                       tail_rows * static_cast<double>(n_cols) * 4.0 * (2.0 * ks) / 8.25e6 + 6.0;
  if (split < whole * 0.99) best = TailSplit{m1 * kTileM, ks};
  return best;
}

BwdPlan plan_bwd(int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t n, size_t esize,
                 void* ws) {
  (void)V_real;
  BwdPlan p{};
  p.S = V_pad / n;
  p.n = n;
  // At least two chunks once the table spans two tiles (G is never staged for
  // the whole vocabulary), more when a chunk would pass kChunkRows rows.
  // Whole shards are grouped into equal chunks when they fit; otherwise
  // every shard is cut into tile-aligned pieces.
  const int64_t want = V_pad >= 2 * kTileM ? max(int64_t{2}, cdiv(V_pad, kChunkRows)) : 1;
  if (want <= n) {
    p.group = cdiv(n, want);
    p.n_chunks = cdiv(n, p.group);
    p.pieces = 1;
    p.piece_rows = p.S;
    p.chunk_rows = p.group * p.S;
  } else {
    p.group = 0;
    const int64_t per = cdiv(want, n);
    p.piece_rows = min(p.S, round_up(cdiv(p.S, per), kTileM));
    p.pieces = cdiv(p.S, p.piece_rows);
    p.n_chunks = p.pieces * n;
    p.chunk_rows = p.piece_rows;
  }
  p.ldC = round_up(p.chunk_rows, kPadK);
  p.esize = esize;
  // K splits: dh has cdiv(T, 256) x cdiv(H, 256) tiles over the chunk's
  // classes, dW cdiv(chunk, 256) x cdiv(H, 256) tiles over the tokens
  const int64_t tiles_h = cdiv(H, kTileN);
  p.split_dh = k_splits_for(cdiv(T, kTileM) * tiles_h, p.chunk_rows, T * H);
  p.split_dw = k_splits_for(cdiv(p.chunk_rows, kTileM) * tiles_h, T, p.chunk_rows * H);
  Carve c(ws);
  p.G = c.take<char>(static_cast<size_t>(T * p.ldC) * esize);
  p.Pdh = c.take<float>(static_cast<size_t>((p.split_dh - 1) * T * H));
  p.Pdw = c.take<float>(static_cast<size_t>((p.split_dw - 1) * p.chunk_rows * H));
  p.dw_tail = p.split_dw == 1 ? tail_split_for(p.chunk_rows, tiles_h, T, H)
                              : TailSplit{p.chunk_rows, 1};
  p.Pdw_tail = c.take<float>(
      static_cast<size_t>((p.dw_tail.ks - 1) * (p.chunk_rows - p.dw_tail.m1) * H));
  p.bytes = c.used;
  return p;
}

// ------------------------------------------------------------------ kernels

// Per token: merge the tile statistics of each shard into (m_k, s_k), then
// the shards into the global log-sum-exp; loss = lse - target logit for
// valid targets. A workgroup takes 32 tokens; 8 lane groups each merge every
// 8th tile of a shard, and the 8 partial pairs are merged in group order, so
// the result does not depend on scheduling. Block partial sums of the loss
// and the counts follow in a fixed shuffle-tree order.
__global__ __launch_bounds__(256) void k_ce_merge(
    const float2* __restrict__ stats, const float* __restrict__ zt,
    const int32_t* __restrict__ targets, int64_t T, int64_t V_real, int32_t ignore_index,
    const SegTable sg, float* __restrict__ lse, float* __restrict__ loss,
    float* __restrict__ shard_stats, float* __restrict__ part_loss,
    int32_t* __restrict__ part_nv, int32_t* __restrict__ part_nb) {
  constexpr int NSUB = 256 / kMergeTok;
  __shared__ float2 red[NSUB][kMergeTok];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok = lane & (kMergeTok - 1);
  const int sub = wave * 2 + (lane >> 5);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kMergeTok + tok;
  const bool tin = t < T;
  float M = -INFINITY, Ssum = 0.0f;
  const int32_t n_seg = sg.n;
  for (int32_t k = 0; k < n_seg; ++k) {
    float mk = -INFINITY, sk = 0.0f;
    const int64_t tiles_per_seg = sg.tile[k + 1] - sg.tile[k];
    if (tin) {
      const float2* st = stats + static_cast<int64_t>(sg.tile[k]) * T + t;
      int64_t j = sub;
      for (; j + 3 * NSUB < tiles_per_seg; j += 4 * NSUB) {
        const float2 v0 = st[j * T];
        const float2 v1 = st[(j + NSUB) * T];
        const float2 v2 = st[(j + 2 * NSUB) * T];
        const float2 v3 = st[(j + 3 * NSUB) * T];
        lse_merge(mk, sk, v0.x, v0.y);
        lse_merge(mk, sk, v1.x, v1.y);
        lse_merge(mk, sk, v2.x, v2.y);
        lse_merge(mk, sk, v3.x, v3.y);
      }
      for (; j < tiles_per_seg; j += NSUB) {
        const float2 v = st[j * T];
        lse_merge(mk, sk, v.x, v.y);
      }
    }
    red[sub][tok] = make_float2(mk, sk);
    __syncthreads();
    if (sub == 0 && tin) {
#pragma unroll
      for (int w = 1; w < NSUB; ++w) lse_merge(mk, sk, red[w][tok].x, red[w][tok].y);
      if (shard_stats) {
        shard_stats[static_cast<int64_t>(k) * T + t] = mk;
        shard_stats[static_cast<int64_t>(n_seg + k) * T + t] = sk;
      }
      lse_merge(M, Ssum, mk, sk);
    }
    __syncthreads();
  }
  if (sub != 0) return;  // lanes 0..31 of wave 0 finish the tokens
  float l = 0.0f;
  int32_t nv = 0, nb = 0;
  if (tin) {
    const float L = M + logf(Ssum);
    lse[t] = L;
    const int64_t y = targets[t];
    const bool valid = (y >= 0) && (y < V_real);
    const bool bad = !valid && (y != ignore_index);
    l = valid ? (L - zt[t]) : 0.0f;
    loss[t] = l;
    nv = valid ? 1 : 0;
    nb = bad ? 1 : 0;
  }
#pragma unroll
  for (int o = kMergeTok / 2; o > 0; o >>= 1) {
    l += __shfl_xor(l, o);
    nv += __shfl_xor(nv, o);
    nb += __shfl_xor(nb, o);
  }
  if (lane == 0) {
    part_loss[blockIdx.x] = l;
    part_nv[blockIdx.x] = nv;
    part_nb[blockIdx.x] = nb;
  }
}

__global__ __launch_bounds__(256) void k_ce_finalize(const float* __restrict__ part_loss,
                                                     const int32_t* __restrict__ part_nv,
                                                     const int32_t* __restrict__ part_nb,
                                                     int64_t nparts, float* loss_sum,
                                                     int32_t* n_valid, int32_t* n_bad) {
  __shared__ float s_l[256];
  __shared__ int32_t s_v[256], s_b[256];
  float l = 0.0f;
  int32_t nv = 0, nb = 0;
  for (int64_t i = threadIdx.x; i < nparts; i += 256) {
    l += part_loss[i];
    nv += part_nv[i];
    nb += part_nb[i];
  }
  s_l[threadIdx.x] = l;
  s_v[threadIdx.x] = nv;
  s_b[threadIdx.x] = nb;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) {
      s_l[threadIdx.x] += s_l[threadIdx.x + w];
      s_v[threadIdx.x] += s_v[threadIdx.x + w];
      s_b[threadIdx.x] += s_b[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *loss_sum = s_l[0];
    *n_valid = s_v[0];
    *n_bad = s_b[0];
  }
}

// (v, i) beats (bv, bi): a larger value, or an equal value at a lower index
// (-1 marks "no row"). A total order, so any merge order gives one result.
__device__ __forceinline__ void argmax_merge(float& bv, int32_t& bi, float v, int32_t i) {
  if (v > bv || (v == bv && i >= 0 && (bi < 0 || i < bi))) {
    bv = v;
    bi = i;
  }
}

// Per token: the tile reports of each shard merged into the shard's report
// (what one rank would hold), then the shard reports into the global argmax.
// 32 tokens per workgroup, 8 lane groups over every 8th tile of a shard.
__global__ __launch_bounds__(256) void k_argmax_merge(
    const float* __restrict__ val, const int32_t* __restrict__ idx, int64_t T,
    const SegTable sg, int32_t* __restrict__ index, float* __restrict__ value,
    float* __restrict__ shard_value, int32_t* __restrict__ shard_index) {
  constexpr int NSUB = 256 / kMergeTok;
  __shared__ float rv[NSUB][kMergeTok];
  __shared__ int32_t ri[NSUB][kMergeTok];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok = lane & (kMergeTok - 1);
  const int sub = wave * 2 + (lane >> 5);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kMergeTok + tok;
  const bool tin = t < T;
  float gv = -INFINITY;
  int32_t gi = -1;
  for (int32_t k = 0; k < sg.n; ++k) {
    float bv = -INFINITY;
    int32_t bi = -1;
    const int64_t tiles_per_seg = sg.tile[k + 1] - sg.tile[k];
    if (tin) {
      const int64_t base = static_cast<int64_t>(sg.tile[k]) * T + t;
      for (int64_t j = sub; j < tiles_per_seg; j += NSUB)
        argmax_merge(bv, bi, val[base + j * T], idx[base + j * T]);
    }
    rv[sub][tok] = bv;
    ri[sub][tok] = bi;
    __syncthreads();
    if (sub == 0 && tin) {
#pragma unroll
      for (int w = 1; w < NSUB; ++w) argmax_merge(bv, bi, rv[w][tok], ri[w][tok]);
      if (shard_value) shard_value[static_cast<int64_t>(k) * T + t] = bv;
      if (shard_index) shard_index[static_cast<int64_t>(k) * T + t] = bi;
      argmax_merge(gv, gi, bv, bi);
    }
    __syncthreads();
  }
  if (sub == 0 && tin) {
    index[t] = gi;
    value[t] = gv;
  }
}

__global__ void k_fill_scalars(float* f0, int32_t* i0, int32_t* i1) {
  if (threadIdx.x == 0) {
    if (f0) *f0 = 0.0f;
    if (i0) *i0 = 0;
    if (i1) *i1 = 0;
  }
}

// G[t][v] = 0 for v in [c0, c1) (columns of the staged G past the chunk)
template <typename E>
__global__ void k_zero_cols(E* G, int64_t rows, int64_t ld, int64_t c0, int64_t c1) {
  const int64_t w = c1 - c0;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < rows * w) G[(i / w) * ld + c0 + i % w] = E(0);
}

// C[r][:] += P[0][r][:] + P[1][r][:] + ... for rows r < rows, planes in order
// (the partial sums of the later K splits; deterministic).
__global__ __launch_bounds__(256) void k_split_add(float* __restrict__ C, int64_t ldc,
                                                   const float* __restrict__ P, int64_t ldp,
                                                   int64_t plane, int32_t nplanes, int64_t rows,
                                                   int64_t cols4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * cols4) return;
  const int64_t r = i / cols4, c = (i - r * cols4) * 4;
  float4* dst = reinterpret_cast<float4*>(C + r * ldc + c);
  float4 v = *dst;
  for (int32_t k = 0; k < nplanes; ++k) {
    const float4 a = *reinterpret_cast<const float4*>(P + k * plane + r * ldp + c);
    v.x += a.x;
    v.y += a.y;
    v.z += a.z;
    v.w += a.w;
  }
  *dst = v;
}

__global__ __launch_bounds__(256) void k_zero_f4(float4* __restrict__ p, int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ------------------------------------------------------------------ launchers

// Persistent launch: one workgroup per CU (a multiple of 8, one group of
// workgroups per XCD), never more than there are tiles (rounded up to 8).
static int64_t persistent_blocks(int64_t tiles) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 8)
    cus = 256;
  const int64_t grid = static_cast<int64_t>(cus / 8) * 8 * kOcc;
  return min(grid, round_up(tiles, 8));
}

// K staging of each GEMM: bytes per operand position per K slice, LDS
// stages, and whether a slice's loads are spread over the MFMAs of the slice
// two before its use (needs three or more stages) or issued together right
// after the barrier that frees their stage.
struct Staging {
  int rb, ns;
  bool spread;
};
template <int MODE, bool AKM, bool BKM>
constexpr Staging staging() {
  if constexpr (MODE == EPI_FWD || MODE == EPI_ARGMAX)
    return {VCE_FWD_RB, VCE_FWD_NS, VCE_FWD_SPREAD != 0};
  else if constexpr (MODE == EPI_GRAD) return {VCE_GRAD_RB, VCE_GRAD_NS, VCE_GRAD_SPREAD != 0};
  else if constexpr (!AKM) return {VCE_DH_RB, VCE_DH_NS, VCE_DH_SPREAD != 0};
  else return {VCE_DW_RB, VCE_DW_NS, VCE_DW_SPREAD != 0};
}

template <typename E, int MODE, bool AKM = false, bool BKM = false>
static hipError_t launch_gemm(const GemmShape& g, const EpiArgs& e, hipStream_t s) {
  const int64_t tiles = static_cast<int64_t>(g.seg.tile[g.seg.n]) * g.tiles_n * g.k_splits;
  if (tiles <= 0) return hipSuccess;
  if (tiles >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const int64_t blocks = persistent_blocks(tiles);
  constexpr Staging st = staging<MODE, AKM, BKM>();
  hipLaunchKernelGGL((k_gemm_tn<E, MODE, AKM, BKM, kTileM, kTileN, kWavesM, kWavesN, st.rb, st.ns,
                                kOcc, st.spread>),
                     dim3(static_cast<uint32_t>(blocks)), dim3(64 * kWavesM * kWavesN), 0, s, g, e);
  return hipGetLastError();
}

hipError_t run_fill_scalars(float* f0, int32_t* i0, int32_t* i1, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_scalars, dim3(1), dim3(64), 0, s, f0, i0, i1);
  return hipGetLastError();
}

hipError_t run_ce_fwd(const void* h, const void* W, const int32_t* targets, int64_t T, int64_t H,
                      int64_t V_real, int64_t V_pad, int32_t ignore_index, bool bf16,
                      float* lse, float* loss, float* loss_sum, int32_t* n_valid, int32_t* n_bad,
                      float* shard_stats, const FwdPlan& p, hipStream_t s) {
  if (T == 0) return run_fill_scalars(loss_sum, n_valid, n_bad, s);
  GemmShape g{};
  g.A = W;
  g.lda = H;
  g.B = h;
  g.ldb = H;
  g.seg = p.seg;
  g.m_total = V_pad;
  g.m_load_end = V_real;
  g.n_total = T;
  g.tiles_n = static_cast<int32_t>(p.tiles_n);
  g.k_splits = 1;
  g.k_total = H;
  g.k_per_split = round_up(H, kPadK);
  g.group_m = kGroupM;
  EpiArgs e{};
  e.fwd.targets = targets;
  e.fwd.T = T;
  e.fwd.V_real = V_real;
  e.fwd.stats = p.stats;
  e.fwd.zt = p.zt;
  hipError_t err = bf16 ? launch_gemm<uint16_t, EPI_FWD>(g, e, s) : launch_gemm<float, EPI_FWD>(g, e, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_ce_merge, dim3(static_cast<uint32_t>(p.merge_blocks)), dim3(256), 0, s,
                     p.stats, p.zt, targets, T, V_real, ignore_index, p.seg, lse,
                     loss, shard_stats, p.part_loss, p.part_nv, p.part_nb);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_ce_finalize, dim3(1), dim3(256), 0, s, p.part_loss, p.part_nv, p.part_nb,
                     p.merge_blocks, loss_sum, n_valid, n_bad);
  return hipGetLastError();
}

hipError_t run_argmax(const void* h, const void* W, int64_t T, int64_t H, int64_t V_real,
                      int64_t V_pad, bool bf16, int32_t* index, float* value,
                      float* shard_value, int32_t* shard_index, const ArgPlan& p,
                      hipStream_t s) {
  if (T == 0) return hipSuccess;
  GemmShape g{};
  g.A = W;
  g.lda = H;
  g.B = h;
  g.ldb = H;
  g.seg = p.seg;
  g.m_total = V_pad;
  g.m_load_end = V_real;
  g.n_total = T;
  g.tiles_n = static_cast<int32_t>(p.tiles_n);
  g.k_splits = 1;
  g.k_total = H;
  g.k_per_split = round_up(H, kPadK);
  g.group_m = kGroupM;
  EpiArgs e{};
  e.arg.T = T;
  e.arg.val = p.val;
  e.arg.idx = p.idx;
  hipError_t err =
      bf16 ? launch_gemm<uint16_t, EPI_ARGMAX>(g, e, s) : launch_gemm<float, EPI_ARGMAX>(g, e, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_argmax_merge, dim3(static_cast<uint32_t>(cdiv(T, kMergeTok))), dim3(256), 0,
                     s, p.val, p.idx, T, p.seg, index, value, shard_value,
                     shard_index);
  return hipGetLastError();
}

template <typename E>
static hipError_t ce_bwd_impl(const void* h, const void* W, const int32_t* targets,
                              const float* lse, const float* grad_loss, const int32_t* n_valid,
                              int32_t reduction, int64_t T, int64_t H, int64_t V_real,
                              int64_t V_pad, int32_t n, float* dh, float* dW, int32_t accumulate,
                              const BwdPlan& p, hipStream_t s, void* const* ev) {
  (void)V_pad;
  (void)n;
  const bool acc_dw = (accumulate & 1) != 0, acc_dh = (accumulate & 2) != 0;
  hipError_t err;
  int ev_i = 0;
  auto mark = [&]() -> hipError_t {
    return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[ev_i++]), s) : hipSuccess;
  };
  auto zero_rows = [&](int64_t r0, int64_t r1) -> hipError_t {  // dW rows [r0, r1) = 0
    const int64_t n4 = (r1 - r0) * H / 4;
    if (n4 <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero_f4, dim3(static_cast<uint32_t>(cdiv(n4, 256))), dim3(256), 0, s,
                       reinterpret_cast<float4*>(dW + r0 * H), n4);
    return hipGetLastError();
  };
  // adds the partial planes of K splits 1.. into rows [0, rows_real) of C
  auto split_add = [&](float* C, const float* P, int32_t ks, int64_t rows,
                       int64_t rows_real) -> hipError_t {
    if (ks <= 1 || rows_real <= 0) return hipSuccess;
    const int64_t cols4 = H / 4;
    const int64_t n = rows_real * cols4;
    hipLaunchKernelGGL(k_split_add, dim3(static_cast<uint32_t>(cdiv(n, 256))), dim3(256), 0, s, C,
                       H, P, H, rows * H, ks - 1, rows_real, cols4);
    return hipGetLastError();
  };
  if ((err = mark()) != hipSuccess) return err;
  const E* Wp = static_cast<const E*>(W);
  E* Gc = static_cast<E*>(p.G);
  bool dh_written = false;
  int32_t dh_planes = 0;    // partial planes of dh that hold sums of earlier chunks
  int64_t last_real = 0;    // the last chunk with a real class: it adds the planes into dh
  for (int64_t c = 0; c < p.n_chunks; ++c) {
    int64_t c0, c1;
    p.chunk(c, c0, c1);
    if (c0 < V_real) last_real = c;
  }
  for (int64_t c = 0; c < p.n_chunks; ++c) {
    int64_t c0, c1;
    p.chunk(c, c0, c1);
    const int64_t Vc = c1 - c0;
    const int64_t kreal = max(min(V_real - c0, Vc), int64_t{0});  // real classes in the chunk
    if (T == 0 || kreal == 0) {
      // no token, or no real class: G is zero, nothing reaches dh, the rows of dW are 0
      if (!acc_dw && (err = zero_rows(c0, c1)) != hipSuccess) return err;
      for (int i = 0; i < 3; ++i)
        if ((err = mark()) != hipSuccess) return err;
      continue;
    }
    // 1. G chunk = scale * (softmax - onehot) over vocabulary rows [c0, c1)
    {
      const int64_t pad_end = min(round_up(Vc, 16 / static_cast<int64_t>(sizeof(E))), p.ldC);
      if (pad_end > Vc) {  // the chunk of G that straddles Vc is read whole
        const int64_t cnt = T * (pad_end - Vc);
        hipLaunchKernelGGL(k_zero_cols<E>, dim3(static_cast<uint32_t>(cdiv(cnt, 256))), dim3(256),
                           0, s, Gc, T, p.ldC, Vc, pad_end);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
      GemmShape g{};
      g.A = Wp + c0 * H;
      g.lda = H;
      g.B = h;
      g.ldb = H;
      g.seg = one_segment(Vc);
      g.m_total = Vc;
      g.m_load_end = kreal;
      g.n_total = T;
      g.tiles_n = static_cast<int32_t>(cdiv(T, kTileN));
      g.k_splits = 1;
      g.k_total = H;
      g.k_per_split = round_up(H, kPadK);
      g.group_m = kGroupM;
      EpiArgs e{};
      e.grad.targets = targets;
      e.grad.lse = lse;
      e.grad.T = T;
      e.grad.V_real = V_real;
      e.grad.grad_loss = grad_loss;
      e.grad.n_valid = n_valid;
      e.grad.v_off = c0;
      e.grad.reduction = reduction;
      e.grad.vec_store = 1;  // tiles start at multiples of 256 rows; ldC is a multiple of 64
      e.grad.G = Gc;
      e.grad.ldG = p.ldC;
      if ((err = launch_gemm<E, EPI_GRAD>(g, e, s)) != hipSuccess) return err;
    }
    if ((err = mark()) != hipSuccess) return err;
    // 2. dh (+)= G W_chunk  (K = the chunk's real classes; W read K-major)
    {
      GemmShape g{};
      g.A = Gc;
      g.lda = p.ldC;
      g.B = Wp + c0 * H;
      g.ldb = H;
      g.seg = one_segment(T);
      g.m_total = T;
      g.m_load_end = T;
      g.n_total = H;
      g.tiles_n = static_cast<int32_t>(cdiv(H, kTileN));
      const int32_t ks = min(k_splits_for(cdiv(T, kTileM) * g.tiles_n, kreal, T * H), p.split_dh);
      g.k_splits = ks;
      g.k_total = kreal;
      g.k_per_split = round_up(cdiv(kreal, ks), kPadK);
      g.group_m = kGroupMdh;
      EpiArgs e{};
      e.store.C = dh;
      e.store.ldc = H;
      e.store.P = p.Pdh;
      e.store.split_stride = T * H;
      e.store.accumulate = (dh_written || acc_dh) ? 1 : 0;
      e.store.planes_held = dh_planes;  // later chunks add into the planes of earlier ones
      e.store.m_zero_from = T;
      if ((err = launch_gemm<E, EPI_STORE, false, true>(g, e, s)) != hipSuccess) return err;
      dh_planes = max(dh_planes, ks - 1);
      // the planes are added into dh once, after the last real chunk's dh
      if (c == last_real && (err = split_add(dh, p.Pdh, dh_planes + 1, T, T)) != hipSuccess)
        return err;
      dh_written = true;
    }
    if ((err = mark()) != hipSuccess) return err;
    // 3. dW rows [c0, c1) = G^T h  (K = tokens; G and h read K-major);
    //    rows of padding classes receive 0 (or are left alone when accumulating).
    //    Rows [r0, r1) of the chunk in one launch of ks K splits, planes at P.
    auto dw_rows = [&](int64_t r0, int64_t r1, int32_t ks, float* P) -> hipError_t {
      GemmShape g{};
      g.A = Gc + r0;
      g.lda = p.ldC;
      g.B = h;
      g.ldb = H;
      g.seg = one_segment(r1 - r0);
      g.m_total = r1 - r0;
      g.m_load_end = r1 - r0;
      g.n_total = H;
      g.tiles_n = static_cast<int32_t>(cdiv(H, kTileN));
      g.k_splits = ks;
      g.k_total = T;
      g.k_per_split = round_up(cdiv(T, ks), kPadK);
      g.group_m = kGroupMdw;
      EpiArgs e{};
      e.store.C = dW + (c0 + r0) * H;
      e.store.ldc = H;
      e.store.P = P;
      e.store.split_stride = (r1 - r0) * H;
      e.store.accumulate = acc_dw ? 1 : 0;
      e.store.m_zero_from = max(kreal - r0, int64_t{0});
      hipError_t er = launch_gemm<E, EPI_STORE, true, true>(g, e, s);
      if (er != hipSuccess) return er;
      return split_add(dW + (c0 + r0) * H, P, ks, r1 - r0, max(kreal - r0, int64_t{0}));
    };
    {
      const int64_t tiles_h = cdiv(H, kTileN);
      const int32_t ks = min(k_splits_for(cdiv(Vc, kTileM) * tiles_h, T, Vc * H), p.split_dw);
      // the last partial round of an unsplit launch split in K, when the
      // plane workspace planned for a whole chunk holds it
      TailSplit ts{Vc, 1};
      if (ks == 1 && p.dw_tail.ks > 1) {
        ts = tail_split_for(Vc, tiles_h, T, H);
        if (ts.ks > 1 && (ts.ks - 1) * (Vc - ts.m1) >
                             (p.dw_tail.ks - 1) * (p.chunk_rows - p.dw_tail.m1))
          ts = TailSplit{Vc, 1};
      }
      if ((err = dw_rows(0, ts.m1, ks, p.Pdw)) != hipSuccess) return err;
      if (ts.m1 < Vc && (err = dw_rows(ts.m1, Vc, ts.ks, p.Pdw_tail)) != hipSuccess) return err;
    }
    if ((err = mark()) != hipSuccess) return err;
  }
  if (T > 0 && !dh_written && !acc_dh) {
    // no real class at all cannot happen (V_real >= 1), but keep dh defined
    const int64_t n4 = T * H / 4;
    hipLaunchKernelGGL(k_zero_f4, dim3(static_cast<uint32_t>(cdiv(n4, 256))), dim3(256), 0, s,
                       reinterpret_cast<float4*>(dh), n4);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t run_ce_bwd(const void* h, const void* W, const int32_t* targets, const float* lse,
                      const float* grad_loss, const int32_t* n_valid, int32_t reduction,
                      int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t n, bool bf16,
                      float* dh, float* dW, int32_t accumulate, const BwdPlan& p, hipStream_t s,
                      void* const* events) {
  if (bf16)
    return ce_bwd_impl<uint16_t>(h, W, targets, lse, grad_loss, n_valid, reduction, T, H, V_real,
                                 V_pad, n, dh, dW, accumulate, p, s, events);
  return ce_bwd_impl<float>(h, W, targets, lse, grad_loss, n_valid, reduction, T, H, V_real, V_pad,
                            n, dh, dW, accumulate, p, s, events);
}

}  // namespace vce
