// One MFMA GEMM core for every contraction of the path:
//     C[m, n] = sum_k A[m, k] * B[n, k]     (both operands K-contiguous)
// with three epilogues:
//   EPI_FWD   logits tile -> per-token (max, sum exp) over the tile's real
//             vocabulary rows + the target logit from the owning tile
//   EPI_GRAD  logits tile -> G = scale * (softmax - onehot), stored twice
//             (token-major and vocabulary-major) in the input element type
//   EPI_STORE plain float32 store / accumulate (dh and dW)
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid over a BM x BN tile; each
// wave owns a (BM/2) x (BN/2) sub-tile made of 32 x 32 MFMA blocks. K advances
// in 128-byte slices (64 bf16 or 32 float), staged in LDS by direct
// global->LDS loads (global_load_lds_dwordx4), two stages deep. Each LDS row
// holds one 128-byte K slice of one operand row, its 16-byte chunks permuted
// by an XOR of the row index so that the fragment reads of 32 consecutive
// rows spread over all banks.
//
// The M side can be cut into equal segments (the vocabulary shards): tiles
// never cross a segment end, so every tile computes with one shard's rows.
#pragma once

#include "vce_device.hpp"

namespace vce {

enum EpiMode { EPI_FWD = 0, EPI_GRAD = 1, EPI_STORE = 2 };

struct GemmShape {
  const void* A;
  int64_t lda;          // elements between consecutive A rows
  const void* B;
  int64_t ldb;
  int64_t seg_len;      // rows per M segment
  int32_t n_seg;        // number of M segments
  int32_t tiles_per_seg;
  int64_t m_total;      // tile ends are clipped to this
  int64_t m_load_end;   // A rows at or past this are never read (loaded as zeros)
  int64_t n_total;      // B rows at or past this are never read
  int32_t tiles_n;
  int32_t k_splits;     // split of K into independent partial products
  int64_t k_total;      // K extent in elements (a multiple of the 16-byte chunk)
  int64_t k_per_split;  // multiple of the K slice
  int32_t group_m;      // tiles along M visited together by one XCD
};

struct FwdArgs {
  const int32_t* targets;
  int64_t T;
  int64_t V_real;
  float2* stats;        // [tiles_m][T]: (max, sum exp(z - max)) of every tile
  float* zt;            // [T]: target logit, written by the owning tile only
};

struct GradArgs {
  const int32_t* targets;
  const float* lse;
  int64_t T;
  int64_t V_real;
  const float* grad_loss;
  const int32_t* n_valid;
  int32_t reduction;    // 0 mean over valid tokens, 1 sum
  int32_t vec_store;    // 1 if every tile start is a multiple of 4 columns
  void* G;              // [T][ldG]
  int64_t ldG;
  void* GT;             // [V rows][ldGT]; columns T..ldGT-1 receive 0
  int64_t ldGT;
};

struct StoreArgs {
  float* C;
  int64_t ldc;
  int64_t split_stride; // elements between split-K partial planes
  int32_t accumulate;   // 1: C += result, 0: C = result
  int64_t m_zero_from;  // rows at or past this receive 0 (or are left alone when accumulating)
};

struct EpiArgs {
  FwdArgs fwd;
  GradArgs grad;
  StoreArgs store;
};

// 16 zero bytes: the source of every masked chunk (rows or K past the end)
static __device__ __attribute__((aligned(64))) const uint32_t g_zero_chunk[16] = {0};

template <typename E>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16 bits
  static constexpr int kSlice = 64;  // elements per 128-byte K slice
  static constexpr int kChunk = 8;   // elements per 16-byte chunk
};
template <>
struct Elem<float> {
  static constexpr int kSlice = 32;
  static constexpr int kChunk = 4;
};

// chunk permutation of LDS row `row`
__device__ __forceinline__ int lds_swz(int row) { return row & 7; }

template <typename E>
__device__ __forceinline__ void mma_chunk(f32x16& acc, const u32x4& a, const u32x4& b);

template <>
__device__ __forceinline__ void mma_chunk<uint16_t>(f32x16& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// float32: the lane's 4 floats are 4 K positions; one 32x32x2 MFMA per
// component (lanes 0-31 give one K position, lanes 32-63 another). A and B
// use the same assignment, so the four products cover the 8 K values of the
// two chunks once each.
template <>
__device__ __forceinline__ void mma_chunk<float>(f32x16& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Stage ROWS operand rows x one 128-byte K slice into LDS at `dst`.
// Wave w moves rows [(q*4 + w)*8, +8) for q = 0..ROWS/32-1: lane l brings the
// 16-byte chunk (l & 7) ^ swz(row) of row (l >> 3), written to LDS at
// dst + row*128 + (l & 7)*16 (the LDS side of these loads is lane-linear).
template <typename E, int ROWS>
__device__ __forceinline__ void stage_rows(char* dst, const E* src, int64_t ld, int64_t row0,
                                           int64_t row_end, int64_t k, int64_t k_end,
                                           int wave, int lane) {
  constexpr int EPC = Elem<E>::kChunk;
#pragma unroll
  for (int q = 0; q < ROWS / 32; ++q) {
    const int r0 = (q * 4 + wave) * 8;
    const int row = r0 + (lane >> 3);
    const int lch = (lane & 7) ^ lds_swz(row);
    const int64_t grow = row0 + row;
    const int64_t gk = k + static_cast<int64_t>(lch) * EPC;
    const void* p = (grow < row_end && gk < k_end)
                        ? static_cast<const void*>(src + grow * ld + gk)
                        : static_cast<const void*>(g_zero_chunk);
    __builtin_amdgcn_global_load_lds(p, (lds_ptr_t)(dst + r0 * 128), 16, 0, 0);
  }
}

template <typename E, int MODE, int BM, int BN>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void k_gemm_tn(GemmShape g, EpiArgs e) {
  constexpr int BK = Elem<E>::kSlice;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int STAGE = A_BYTES + B_BYTES;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sizes");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;

  // ---- which tile
  const int64_t tiles_m = static_cast<int64_t>(g.n_seg) * g.tiles_per_seg;
  const int64_t per_split = tiles_m * g.tiles_n;
  const int64_t total = per_split * g.k_splits;
  const int64_t L = xcd_logical_block(blockIdx.x, total);
  const int64_t ks = L / per_split;
  const int64_t rem = L - ks * per_split;
  const int64_t in_group = static_cast<int64_t>(g.group_m) * g.tiles_n;
  const int64_t grp = rem / in_group;
  const int64_t first_m = grp * g.group_m;
  const int64_t gsz = min(static_cast<int64_t>(g.group_m), tiles_m - first_m);
  const int64_t r_in = rem - grp * in_group;
  const int64_t tm = first_m + r_in % gsz;
  const int64_t tn = r_in / gsz;
  const int64_t seg = tm / g.tiles_per_seg;
  const int64_t tj = tm - seg * g.tiles_per_seg;
  const int64_t m0 = seg * g.seg_len + tj * BM;
  const int64_t m_end = min(min(m0 + BM, (seg + 1) * g.seg_len), g.m_total);
  const int64_t m_load = min(m_end, g.m_load_end);
  const int64_t n0 = tn * BN;
  const int64_t n_end = min(n0 + static_cast<int64_t>(BN), g.n_total);
  const int64_t k_beg = ks * g.k_per_split;
  const int64_t k_end = min(k_beg + g.k_per_split, g.k_total);

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const E* Ap = static_cast<const E*>(g.A);
  const E* Bp = static_cast<const E*>(g.B);

  if (m_load > m0 && k_end > k_beg) {
    const int nk = static_cast<int>((k_end - k_beg + BK - 1) / BK);
    stage_rows<E, BM>(smem, Ap, g.lda, m0, m_load, k_beg, k_end, wave, lane);
    stage_rows<E, BN>(smem + A_BYTES, Bp, g.ldb, n0, n_end, k_beg, k_end, wave, lane);
    asm volatile("" ::"r"(smem) : "memory");
    for (int kt = 0; kt < nk; ++kt) {
      __syncthreads();  // stage kt has landed; nobody still reads stage kt+1
      if (kt + 1 < nk) {
        char* nxt = smem + ((kt + 1) & 1) * STAGE;
        const int64_t kk = k_beg + static_cast<int64_t>(kt + 1) * BK;
        stage_rows<E, BM>(nxt, Ap, g.lda, m0, m_load, kk, k_end, wave, lane);
        stage_rows<E, BN>(nxt + A_BYTES, Bp, g.ldb, n0, n_end, kk, k_end, wave, lane);
      }
      asm volatile("" ::"r"(smem) : "memory");
      const char* sA = smem + (kt & 1) * STAGE + wm * WM * 128;
      const char* sB = smem + (kt & 1) * STAGE + A_BYTES + wn * WN * 128;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int ch = ((2 * s + half) ^ lds_swz(l32)) * 16;
        u32x4 a[MI], b[NI];
#pragma unroll
        for (int i = 0; i < MI; ++i)
          a[i] = *reinterpret_cast<const u32x4*>(sA + (i * 32 + l32) * 128 + ch);
#pragma unroll
        for (int j = 0; j < NI; ++j)
          b[j] = *reinterpret_cast<const u32x4*>(sB + (j * 32 + l32) * 128 + ch);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) mma_chunk<E>(acc[i][j], a[i], b[j]);
      }
    }
  }

  // Row of accumulator element r of block i (relative to the wave tile):
  //   i*32 + 8*(r/4) + 4*half + r%4 ;  its column: j*32 + l32.
  const int64_t vbase = m0 + wm * WM;

  if constexpr (MODE == EPI_FWD) {
    const FwdArgs& f = e.fwd;
    const int64_t vend = m_load;  // real rows of this tile end here (m_load_end = V_real)
    const bool full = vbase + WM <= vend;
    __syncthreads();  // all waves are done with the operand stages
    float2* red = reinterpret_cast<float2*>(smem);  // [2][BN]
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t v = vbase + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (full || v < vend) m = fmaxf(m, acc[i][j][r]);
        }
      m = fmaxf(m, __shfl_xor(m, 32));
      float s = 0.0f;
      if (m != -INFINITY) {
        const float mb = m * kLog2e;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t v = vbase + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (full || v < vend) s += fast_exp2(fmaf(acc[i][j][r], kLog2e, -mb));
          }
      }
      s += __shfl_xor(s, 32);
      const int col = wn * WN + j * 32 + l32;
      if (half == 0) red[wm * BN + col] = make_float2(m, s);

      // the owning tile stores the target logit
      const int64_t t = n0 + col;
      const int64_t y = (t < f.T) ? static_cast<int64_t>(f.targets[t]) : -1;
      const bool mine = (y >= vbase) && (y < vbase + WM) && (y < vend);
      if (__any(mine)) {
        const int64_t loc = y - vbase;
        float val = 0.0f;
        bool hit = false;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lr = i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (mine && loc == lr) {
              val = acc[i][j][r];
              hit = true;
            }
          }
        if (hit) f.zt[t] = val;
      }
    }
    __syncthreads();
    if (tid < BN) {
      const int64_t t = n0 + tid;
      if (t < f.T) {
        float2 a = red[tid];
        const float2 b = red[BN + tid];
        lse_merge(a.x, a.y, b.x, b.y);
        f.stats[tm * f.T + t] = a;
      }
    }
  } else if constexpr (MODE == EPI_GRAD) {
    const GradArgs& gr = e.grad;
    const float scale = (gr.reduction == 0)
                            ? gr.grad_loss[0] / static_cast<float>(max(gr.n_valid[0], 1))
                            : gr.grad_loss[0];
    const int64_t vreal_end = min(m_end, gr.V_real);
    E* Gp = static_cast<E*>(gr.G);
    E* GTp = static_cast<E*>(gr.GT);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t t = n0 + wn * WN + j * 32 + l32;
      const bool tin = t < gr.T;
      const int64_t y = tin ? static_cast<int64_t>(gr.targets[t]) : -1;
      const bool valid = tin && y >= 0 && y < gr.V_real;
      const float coef = valid ? scale : 0.0f;
      const float nl = tin ? gr.lse[t] * kLog2e : 0.0f;
      const bool t_gt = t < gr.ldGT;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t v0 = vbase + i * 32 + 8 * q + 4 * half;
          float gv[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int64_t v = v0 + c;
            const float p = fast_exp2(fmaf(acc[i][j][4 * q + c], kLog2e, -nl));
            const float oh = (v == y) ? 1.0f : 0.0f;
            gv[c] = (v < vreal_end) ? coef * (p - oh) : 0.0f;
          }
          if constexpr (sizeof(E) == 2) {
            uint16_t hb[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) hb[c] = f32_to_bf16(gv[c]);
            if (tin) {
              if (gr.vec_store && v0 + 3 < m_end) {
                u32x2 pk;
                pk.x = static_cast<uint32_t>(hb[0]) | (static_cast<uint32_t>(hb[1]) << 16);
                pk.y = static_cast<uint32_t>(hb[2]) | (static_cast<uint32_t>(hb[3]) << 16);
                *reinterpret_cast<u32x2*>(Gp + t * gr.ldG + v0) = pk;
              } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  if (v0 + c < m_end) Gp[t * gr.ldG + v0 + c] = hb[c];
              }
            }
            if (t_gt) {
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (v0 + c < m_end) GTp[(v0 + c) * gr.ldGT + t] = hb[c];
            }
          } else {
            if (tin) {
              if (gr.vec_store && v0 + 3 < m_end) {
                f32x4 pk = {gv[0], gv[1], gv[2], gv[3]};
                *reinterpret_cast<f32x4*>(Gp + t * gr.ldG + v0) = pk;
              } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  if (v0 + c < m_end) Gp[t * gr.ldG + v0 + c] = gv[c];
              }
            }
            if (t_gt) {
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (v0 + c < m_end) GTp[(v0 + c) * gr.ldGT + t] = gv[c];
            }
          }
        }
    }
  } else {  // EPI_STORE
    const StoreArgs& st = e.store;
    float* Cp = st.C + ks * st.split_stride;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = vbase + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (m >= m_end) continue;
        const bool zero_row = m >= st.m_zero_from;
        if (zero_row && st.accumulate) continue;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int64_t n = n0 + wn * WN + j * 32 + l32;
          if (n >= n_end) continue;
          float* dst = Cp + m * st.ldc + n;
          const float v = zero_row ? 0.0f : acc[i][j][r];
          if (st.accumulate)
            *dst += v;
          else
            *dst = v;
        }
      }
  }
}

}  // namespace vce
