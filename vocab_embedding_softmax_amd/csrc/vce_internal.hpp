// Host-side planning shared by the launchers and the C entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vce_device.hpp"

namespace vce {

#ifndef VCE_WAVES_M
#define VCE_WAVES_M 2
#endif
#ifndef VCE_WAVES_N
#define VCE_WAVES_N 4
#endif
#ifndef VCE_TILE_M
#define VCE_TILE_M 256
#endif
#ifndef VCE_TILE_N
#define VCE_TILE_N 256
#endif
#ifndef VCE_OCC
#define VCE_OCC 1
#endif
constexpr int kTileM = VCE_TILE_M;  // GEMM tile rows (M side)
constexpr int kTileN = VCE_TILE_N;  // GEMM tile columns (N side)
constexpr int kOcc = VCE_OCC;       // workgroups resident per CU (waves per SIMD)
#ifndef VCE_CHUNK_ROWS
#define VCE_CHUNK_ROWS 131072
#endif
// K staging per GEMM (bytes per position per K slice, LDS stages, spread
// issue of a slice's loads). Two 128-byte stages everywhere: the bf16 form
// on 16x16x32 blocks needs them, and with 32x32x16 blocks dh and dW ran the
// same with them as with four 64-byte stages.
#ifndef VCE_FWD_RB
#define VCE_FWD_RB 128
#endif
#ifndef VCE_FWD_NS
#define VCE_FWD_NS 2
#endif
#ifndef VCE_FWD_SPREAD
#define VCE_FWD_SPREAD 0
#endif
#ifndef VCE_GRAD_RB
#define VCE_GRAD_RB 128
#endif
#ifndef VCE_GRAD_NS
#define VCE_GRAD_NS 2
#endif
#ifndef VCE_GRAD_SPREAD
#define VCE_GRAD_SPREAD 0
#endif
#ifndef VCE_DH_RB
#define VCE_DH_RB 128
#endif
#ifndef VCE_DH_NS
#define VCE_DH_NS 2
#endif
#ifndef VCE_DH_SPREAD
#define VCE_DH_SPREAD 0
#endif
#ifndef VCE_DW_RB
#define VCE_DW_RB 128
#endif
#ifndef VCE_DW_NS
#define VCE_DW_NS 2
#endif
#ifndef VCE_DW_SPREAD
#define VCE_DW_SPREAD 0
#endif
constexpr int kChunkRows = VCE_CHUNK_ROWS;  // most vocabulary rows of one backward chunk
// Tiles along M that one XCD's 32 workgroups walk together: 4 (4 x 8 tiles
// per round) for the logit GEMMs, 1.5-3 % faster than 2 or 8 there; the dh
// GEMM (T x H tiles) runs 2 % faster with 1 and the dW GEMM (vocabulary x H)
// 1 % faster with 2 than with 4.
#ifndef VCE_GROUP_M
#define VCE_GROUP_M 4
#endif
#ifndef VCE_GROUP_M_DH
#define VCE_GROUP_M_DH 1
#endif
#ifndef VCE_GROUP_M_DW
#define VCE_GROUP_M_DW 2
#endif
constexpr int kGroupM = VCE_GROUP_M;
constexpr int kGroupMdh = VCE_GROUP_M_DH;
constexpr int kGroupMdw = VCE_GROUP_M_DW;
constexpr int kWavesM = VCE_WAVES_M;  // waves per workgroup along M
constexpr int kWavesN = VCE_WAVES_N;  // waves per workgroup along N
constexpr int kPadK = 64;     // staged operands are padded to this many K elements
constexpr int kMergeTok = 32; // tokens per workgroup of the statistics merge
constexpr int kAlign = 256;   // workspace region alignment (bytes)

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Bump allocator over a caller-supplied workspace (or a null base, for sizing).
struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    used = static_cast<size_t>(round_up(static_cast<int64_t>(used), kAlign));
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

// Segments of a table: the given shard row offsets (num_shards + 1 values,
// validated by the caller) or, with none, equal shards of V_pad / n rows;
// tiles of kTileM rows per shard, never crossing a shard end.
SegTable shard_segments(int32_t n, const int64_t* rows, int64_t V_pad);
// One segment of `rows` rows.
SegTable one_segment(int64_t rows);

// Forward cross-entropy plan: vocabulary tiles per shard, token tiles.
struct FwdPlan {
  SegTable seg;
  int64_t tiles_m, tiles_n, merge_blocks;
  float2* stats;
  float* zt;
  float* part_loss;
  int32_t* part_nv;
  int32_t* part_nb;
  size_t bytes;
};
FwdPlan plan_fwd(int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t n,
                 const int64_t* rows, void* ws);

// Greedy argmax plan: per-tile reports (largest logit, its row) of every
// vocabulary tile of every shard, [tiles_m][T] each.
struct ArgPlan {
  SegTable seg;
  int64_t tiles_m, tiles_n;
  float* val;
  int32_t* idx;
  size_t bytes;
};
ArgPlan plan_argmax(int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t n,
                    const int64_t* rows, void* ws);

// Backward plan: the vocabulary is processed in chunks; only one chunk's
// G = [T][chunk] is staged. A chunk is a group of whole shards, or a piece of
// one shard when shards are larger than a chunk may be.
// An unsplit GEMM whose tiles fill their last round of CUs only in part can
// run as two launches: output rows [0, m1) unsplit (the most whole rows of
// tiles that fit in the whole rounds), and rows [m1, rows) with K split in ks
// parts (planes added afterwards), so that the last round's tiles take a
// fraction of a tile's time. ks == 1: one launch.
struct TailSplit {
  int64_t m1;
  int32_t ks;
};
// The split of a GEMM of `rows` output rows (tiles of kTileM), tiles_n tiles
// along N and K positions (n_cols float32 outputs per row), by the same
// estimate as k_splits_for; {rows, 1} when it saves less than 1 %.
TailSplit tail_split_for(int64_t rows, int64_t tiles_n, int64_t K, int64_t n_cols);

struct BwdPlan {
  int64_t S;                 // rows per shard
  int64_t n;                 // shards
  int64_t group;             // shards per chunk (0: chunks are pieces of a shard)
  int64_t pieces;            // chunks per shard (pieces)
  int64_t piece_rows;        // rows per piece (the last piece of a shard may be shorter)
  int64_t chunk_rows;        // most rows of a chunk
  int64_t n_chunks;
  int64_t ldC;               // leading dimension of the staged G chunk
  size_t esize;
  void* G;                   // [T][ldC]
  int32_t split_dh;          // most K splits of the dh GEMM (1: none)
  int32_t split_dw;          // most K splits of the dW GEMM
  float* Pdh;                // [split_dh - 1][T][H] partial planes
  float* Pdw;                // [split_dw - 1][chunk_rows][H]
  TailSplit dw_tail;         // split of the unsplit dW GEMM's last round (chunk_rows rows)
  float* Pdw_tail;           // [dw_tail.ks - 1][chunk_rows - dw_tail.m1][H]
  size_t bytes;
  void chunk(int64_t c, int64_t& c0, int64_t& c1) const {
    if (group > 0) {
      c0 = c * group * S;
      c1 = (c + 1) * group < n ? (c + 1) * group * S : n * S;
      return;
    }
    const int64_t k = c / pieces, j = c % pieces;
    c0 = k * S + j * piece_rows;
    c1 = (k + 1) * S < c0 + piece_rows ? (k + 1) * S : c0 + piece_rows;
  }
};
// K splits for a GEMM of `tiles` output tiles (out_elems float32 outputs)
// over K positions: the count in 1..8 (each split >= 1024 K positions) with
// the least estimated time, rounds of tiles over the GPU's 256 CUs plus the
// partial planes' writes and their addition; a split must save 2 %.
int32_t k_splits_for(int64_t tiles, int64_t K, int64_t out_elems);
BwdPlan plan_bwd(int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t n, size_t esize,
                 void* ws);

// Embedding backward plan: a stable sort of the tokens by ID, then one launch
// of segment sums (short IDs by the chunk of the sorted list where their run
// starts, long IDs by column slices; see vce_emb.hip). Two ways to sort:
//   runs: up to 32768 tokens, runs of 1024 radix-sorted in LDS, then placed
//     by their ranks in every run (two launches);
//   general: block-local LDS sorts + per-block counts + scans (any size).
struct EmbBwdPlan {
  bool runs;           // sorted runs + merge (T <= 32 runs of 1024 tokens), else general
  int32_t vbits;       // bits of an ID
  int64_t nruns;       // runs of 1024 tokens
  int64_t nblocks;     // token blocks of the local sort (general)
  int64_t nchunks, nslices, scan_blocks;
  int32_t* bcnt;       // [nblocks][V_real] per-block occurrences -> per-block offsets (general)
  int32_t* counts;     // [V_real] occurrences of each ID (general)
  int32_t* offs;       // [V_real + 1] exclusive prefix of counts, offs[V_real] = total (general)
  uint64_t* lkey;      // [nblocks * block] block-sorted keys (ID << 32 | token) (general)
  int32_t* lrank;      // [nblocks * block] rank among equal IDs inside the block (general)
  int32_t* scan_tmp;   // [scan_blocks + 1] (general)
  int32_t* sorted;     // [T] token indices sorted by (ID, token)
  int32_t* skey;       // [T] the ID of each sorted position
  uint32_t* rid;       // [nruns * 1024] IDs of each sorted run (all bits set: no valid ID)
  int32_t* rtok;       // [nruns * 1024] their tokens
  int32_t* rvalid;     // [nruns] valid tokens per run
  int32_t* n_sorted;   // [1] number of valid tokens (runs; general: offs + V_real)
  int32_t* chunk_start;// [nchunks] first sorted position of the ID at each chunk's first position
  int32_t* chunk_end;  // [nchunks] one past its last sorted position
  int32_t* long_runs;  // [nchunks][4] (first, end, ID, 0) of every ID with at least kSegLong tokens
  int32_t* n_long;     // [1] number of such IDs
  int64_t long_wgs;    // workgroups of the segment-sum launch that take the long IDs
  size_t bytes;
};
EmbBwdPlan plan_emb_bwd(int64_t T, int64_t H, int64_t V_real, void* ws);

struct CandPlan {
  int64_t scan_blocks_v;
  int32_t* flags;    // [V]
  int32_t* uidx;     // [V + 1]
  int32_t* notin;    // [V]
  int32_t* nidx;     // [V + 1]
  int32_t* scan_tmp; // [scan_blocks + 1]
  size_t bytes;
};
CandPlan plan_cand(int64_t T, int64_t V, void* ws);

// Launchers (all enqueue on `s`; return the first launch error).
hipError_t run_ce_fwd(const void* h, const void* W, const int32_t* targets, int64_t T, int64_t H,
                      int64_t V_real, int64_t V_pad, int32_t ignore_index, bool bf16,
                      float* lse, float* loss, float* loss_sum, int32_t* n_valid, int32_t* n_bad,
                      float* shard_stats, const FwdPlan& p, hipStream_t s);

// events (optional): 1 + 3 * p.n_chunks handles recorded before the first
// kernel and after each chunk's G, dh contribution and dW rows
hipError_t run_ce_bwd(const void* h, const void* W, const int32_t* targets, const float* lse,
                      const float* grad_loss, const int32_t* n_valid, int32_t reduction,
                      int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int32_t n, bool bf16,
                      float* dh, float* dW, int32_t accumulate, const BwdPlan& p, hipStream_t s,
                      void* const* events);

hipError_t run_argmax(const void* h, const void* W, int64_t T, int64_t H, int64_t V_real,
                      int64_t V_pad, bool bf16, int32_t* index, float* value,
                      float* shard_value, int32_t* shard_index, const ArgPlan& p, hipStream_t s);

hipError_t run_emb_fwd(const int32_t* ids, const void* W, int64_t T, int64_t H, int64_t V_real,
                       const SegTable& sg, size_t esize, void* out, int32_t* n_bad,
                       hipStream_t s);

hipError_t run_remap(const int32_t* in, int64_t T, const int32_t* map, int64_t V_real,
                     int32_t* out, hipStream_t s);

hipError_t run_ngram_fwd(const int32_t* ids, const void* E0, const void* E2, const void* E3,
                         int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int64_t rows2,
                         int64_t rows3, int32_t n, bool bf16, void* out, int32_t* ids2,
                         int32_t* ids3, int32_t* n_bad, hipStream_t s);

hipError_t run_emb_bwd(const int32_t* ids, const void* dout, bool dout_bf16, int64_t T, int64_t H,
                       int64_t V_real, int64_t V_pad, float* dW, int32_t accumulate,
                       const EmbBwdPlan& p, hipStream_t s);

// dW[cand[i]] (+)= dWc[i] for distinct cand entries in [0, V); the rest of
// dW zeroed first unless accumulating
hipError_t run_ss_scatter(const int32_t* cand, int64_t P, const float* dWc, int64_t H, int64_t V,
                          float* dW, int32_t accumulate, hipStream_t s);
hipError_t run_ss_scatter_replace(const int32_t* prev, int64_t P_prev, const int32_t* cand,
                                  int64_t P, const float* dWc, int64_t H, int64_t V, float* dW,
                                  hipStream_t s);
hipError_t run_candidates(const int32_t* targets, int64_t T, int64_t V, const int32_t* perm,
                          int64_t P, int32_t* cand, int32_t* pos, int32_t* n_unique,
                          int32_t* n_cand, const CandPlan& p, hipStream_t s);

hipError_t run_fill_scalars(float* f0, int32_t* i0, int32_t* i1, hipStream_t s);

// Static device scratch of the allocation-free argmax: size, and its device
// address on the current device (looked up once per device, then cached).
constexpr size_t kNoAllocScratchBytes = size_t{16} << 20;
hipError_t noalloc_scratch(void** ptr);

// Exclusive scan of n int32 values: y[i] = sum x[0..i), y[n] = total.
// tmp holds scan_blocks(n) + 1 ints.
int64_t scan_blocks(int64_t n);
hipError_t run_scan(const int32_t* x, int64_t n, int32_t* y, int32_t* y_copy, int32_t* tmp,
                    hipStream_t s);

}  // namespace vce
