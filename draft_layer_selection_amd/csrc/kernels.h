// Internal interface between the host driver (knapspec.cpp) and the HIP kernels.
// Not part of the public ABI: argument structs hold device pointers and sizes only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ks {

enum ActType : int { ACT_F32 = 0, ACT_BF16 = 1 };

// ---------------------------------------------------------------------------------------
// GEMM: out[r][n] = sum_k A[r][k] * W[n][k] over the rows of one item (all sequences).
//   mode PARTIAL: fp32 partial sums per K split, P[split][R][ldp]; the consumer adds splits.
//   mode SWIGLU : split must be 1; 64-column tile t holds gate rows [32t, 32t+32) and up
//                 rows [ff + 32t, ...); writes H[r][32t + j] = silu(gate) * up.
// ---------------------------------------------------------------------------------------
enum GemmMode : int { GEMM_PARTIAL = 0, GEMM_SWIGLU = 1 };

constexpr int WIN_MAX = 16;  // largest window r (tokens per DP state or verification block)
constexpr int BEAM_MAX = 8;  // largest beam width (states kept per DP cell)
// largest K-split count of a GEMM; the kernels that add the splits issue one load per split
// before the first addition
constexpr int GEMM_MAX_SPLITS = 16;

struct GemmArgs {
  const void* A;  // [R][lda] activations (bf16 or f32, same as W)
  int lda;
  int R;          // rows
  const void* W;  // [N][K] weights
  int K;
  int N;          // logical output columns (2*ff for SWIGLU)
  int n_tiles;    // N / 64
  int m_tiles;
  int mb;         // 32-row blocks per tile (bf16 kernel), rows per tile = 32*mb
  int splits;
  int k_chunk;    // K per split
  int mode;
  float* P;       // PARTIAL output
  int ldp;
  void* H;        // SWIGLU output
  int ldh;
  int ff;
  int per_xcd;    // ceil(total tiles / 8): XCD-aware tile order
  int ng;         // LDS kernel: 64-column groups per tile (2 or 4); 0 = direct-load kernel
  int areg;       // > 0: activations-in-registers kernel with this many stages of activation
                  // loads in flight (128-column tiles, one tile of up to 256 rows, m_tiles 1)
  const int* amap;    // nullable [R]: A row of output row r is A[amap[r]] (live-row plan)
  const int* r_live;  // nullable device count: m-tiles starting at or past it are skipped
};

// Tile/split plan of one GEMM launch (chosen on the host, see plan_gemm).
struct GemmPlan {
  int ng, mb, m_tiles, n_tiles, splits, k_chunk, areg;
};
GemmPlan plan_gemm(int act, int R, int N, int K, int mode, int ff, size_t cap_floats);
int areg_depth();

// ---------------------------------------------------------------------------------------
// Attention over the shared KV cache (split over context positions) + combine with self.
// ---------------------------------------------------------------------------------------
struct AttnSeq {
  const void* k;  // this layer's K cache of the sequence, [hkv][cap][dh]
  const void* v;
  int ctx;        // cached positions
  int cap;        // positions per head in the buffer
  int row_off;    // first row of the sequence in this item
  int M;          // rows of the sequence in this item (live sources + reference)
  int nsplit;     // context splits
  int chunk;      // positions per split (multiple of 64)
  int part_off;   // first partial slot of the sequence; slot of (split sp, local row r,
                  // head h) = part_off + (sp * M + r) * hq + h
  int pad0;
  int qrows;      // query rows per workgroup of the bf16 MFMA kernel (multiple of 32, at most
                  // 256; 0 = 256): a KV head's G*M query rows are spread evenly over its blocks
  int pad2;
};

// Partial-result slot of one (split, row, query head) of a sequence.
__host__ __device__ inline size_t attn_slot(const AttnSeq& s, int sp, int r_local, int hq,
                                            int h) {
  return (size_t)s.part_off + ((size_t)sp * s.M + r_local) * hq + h;
}

struct AttnArgs {
  const void* Q;       // [R][hq][dh] activations (position-rotated; bf16: times log2(e)/sqrt(dh))
  int hq, hkv, dh;
  const int4* work;    // per workgroup: (seq, kv head, q block, split); seq < 0: no work
  const AttnSeq* seqs; // [n_seqs]
  float* Opart;        // [slots][dh] unnormalised partial outputs
  float* Mpart;        // [slots] running max (log2 domain)
  float* Lpart;        // [slots] partial denominators
  float scale_log2;    // factor from q.k to the log2 domain: log2(e) / sqrt(dh) for float32
                       // (q unscaled); the bf16 MFMA kernel takes q pre-scaled and ignores it
};

struct CombineArgs {
  const void* Q;
  const float* kself;  // [R][hkv][dh]: the item's own keys/values of every row
  const float* vself;
  const int* row_tok;  // [R] window token t of the row: it also attends to the own
                       // keys/values of rows r - t .. r (window tokens 0..t of its state)
  int rmax;            // largest window r of the launch's rows (1: row_tok is not read)
  const float* Opart;
  const float* Mpart;
  const float* Lpart;
  const AttnSeq* seqs;
  const int* row_seq;  // [R]
  int R, hq, hkv, dh;
  float scale_log2;    // q.k to the log2 domain: log2(e)/sqrt(dh) for float32, 1 for bf16 (q pre-scaled)
  void* O;             // [R][hq*dh] activations
};

struct QkvArgs {
  const float* P;      // [splits][R][ldp]
  int splits, R, ldp;
  int hq, hkv, dh;
  const float* rope;   // [n_seqs][wmax][dh]: cos[dh/2] then sin[dh/2] at position ctx + t
  const int* row_seq;  // [R]
  const int* row_tok;  // [R] window token t of the row
  int wmax;
  void* Q;             // [R][hq][dh] activations: the rotated query times q_scale
  float q_scale;       // log2(e)/sqrt(dh) for bf16 (scores come out in the exponent's units), 1 for f32
  float* kself;        // [R][hkv][dh]
  float* vself;
};

// ---------------------------------------------------------------------------------------
// Per-budget cosine / execute-or-skip select (+ RMSNorm of the kept state for the next item).
// ---------------------------------------------------------------------------------------
struct ItemSeq {   // one (item, sequence)
  int w;           // item weight
  int prefix;      // w_0 + ... + w_i
  int row_off;     // first row of the sequence in this item
  int M;           // rows ((sources + reference) x window)
  int ref_row;     // global row of the reference's first token in this item's GEMM output
  int next_ref_row;// same in the next item's activations (-1: none)
  int win;         // r: tokens per state (rows per budget)
  int pad1;
};

// E[r] = state_old[row_state[r]] + sum_s P[s][r]: the item applied to every source row and
// to the reference row (K splits added in a fixed order, then the residual).
struct ReduceArgs {
  const float* P;          // [splits][R][d]
  int splits, R, d;
  const float* state_old;  // [S][Bm+1][d]
  const int* row_state;    // [R] flat index into state_old rows
  float* E;                // [R][d]
};

struct SelectArgs {
  int item, n_items, B, Bm, d, mw, n_seqs;
  int wmax;                // state rows per beam slot (window capacity)
  int rmax;                // largest window r among the solve's sequences
  int kmax;                // beam slots per budget (capacity); valid, masks, exec_row and
                           // next_row hold kmax entries per budget, slot 0 first
  int beam;                // beam width k of this solve (1: the one-state DP)
  const float* E;          // [Rtot][d] item outputs incl. residual (ReduceArgs::E)
  int Rtot;
  const float* state_old;  // [S][Bm+1][kmax][wmax][d], budget index Bm = reference (slot 0)
  float* state_new;
  const uint8_t* valid_old;  // [S][Bm]
  uint8_t* valid_new;
  const uint64_t* mask_old;  // [S][Bm][mw]
  uint64_t* mask_new;
  const int* exec_row;     // [S][Bm] first row of this item whose target budget is b, or -1
  const int* next_row;     // [S][Bm] first row of b in the next item's activations, or -1
  const ItemSeq* info;     // [S]
  float tau;
  int skip_cap;
  float eps;
  void* xa_next;           // [R_next][d] activations of the next item
  int act;                 // ActType of xa_next
  uint8_t* decisions;      // [S][n_items][Bm] or null
  float* margins;          // [S][n_items][Bm] or null
  float* cos_out;          // [S][Bm]
};

// Live-row plan of one DP item (items 1 .. 2L-1), built on the device from the valid flags
// that the previous item's select wrote.  A pruned source budget (tau, skip cap) gets no row:
// sequence q's rows are [live sources in budget order..., reference] x window r, sequences one
// after another.  Launch sizes stay the ones planned from reachability (R_plan rows); rows at
// and past the live count get in-range map entries (sequence 0, token 0, state 0, A row 0) so
// the kernels that process them stay in bounds, and their results are never read.  For an
// attention item it also picks each sequence's context splits for the live rows (the host
// planner's cost model: fewest rounds x (tiles + fixed cost), ties to fewer workgroups, then
// to the earlier candidate) and writes the layer's work list, groups of query blocks dealt to
// the dies round-robin.
constexpr int COMPACT_THREADS = 1024;   // 16 waves, one sequence each; n_budgets <= 1024
constexpr int COMPACT_MAX_SEQS = 64;

struct CompactArgs {
  int n_seqs, B, Bm, kmax, wmax;
  int R_plan;                 // rows the item's launches are sized for
  const uint8_t* valid;       // [S][Bm][kmax] valid flags before this item (slot 0 used)
  const int* prev_next_row;   // previous item's next_row: planned activation row of a source
  const ItemSeq* prev_info;   // previous item's [S] (next_ref_row: planned reference row)
  ItemSeq* info;              // this item's [S]: row_off, M and ref_row rewritten
  int* exec_row;              // this item's [S][Bm][kmax]: entries of candidate sources rewritten
  int* amap;                  // this item's [R_plan] maps
  int* row_seq;
  int* row_tok;
  int* row_state;
  int* r_live;                // out: rows of live sources and references
  // attention item only (aseq == nullptr for an MLP item)
  AttnSeq* aseq;              // the layer's [S]: row_off, M, nsplit, chunk, part_off, qrows
  int4* work;                 // the layer's work list, work_cap entries (-1 = no work)
  int work_cap;
  int hq, hkv, qb_rows, slots, max_split;
  long long part_cap;
};

struct InitArgs {
  int n_seqs, Bm, d, mw, wmax, kmax;
  const float* const* x0;  // device array [n_seqs] of device pointers to [r][d]
  float* state;            // [S][Bm+1][kmax][wmax][d]
  uint8_t* valid;          // [S][Bm][kmax]
  uint64_t* masks;         // [S][Bm][kmax][mw]
  const int* rows;         // [S][4]: first row of budget 0 and of the reference in item 0
                           // (-1 none), the window r, unused
  void* xa;                // item 0 activations
  int act;
  float eps;
};

// Running greedy token of each row over vocabulary chunks: logits of columns
// col0 .. col0+ncols-1 are the K-split partial sums P[s][row][c] (added in split order);
// the best (value, index) replaces the row's running best only when strictly larger, ties
// within a chunk go to the lower index, and NaN logits never win.
struct LmArgmaxArgs {
  const float* P;   // [splits][R][ldp]
  int splits, R, ldp, ncols, col0, first;
  float* best_val;  // [R]
  int* best_idx;    // [R]
};

hipError_t launch_gemm(const GemmArgs& a, int act, hipStream_t s);
hipError_t launch_lm_argmax(const LmArgmaxArgs& a, hipStream_t s);

// Decode-loop helpers (masked draft step and verification):
// carry: for rows t < n, state[t] = src[t] and xa[t] = RMSNorm(src[t]) in the activation type.
hipError_t launch_carry(const float* src, int n, int d, float eps, float* state, void* xa,
                        int act, hipStream_t s);
// embed: out[t] = LM-head row idx[t] (tied embedding), widened to float32, for t < n.
hipError_t launch_embed(const void* w_lm, const int* idx, int n, int d, int act, float* out,
                        hipStream_t s);
// kv_append: the own keys/values of rows t < n (kself/vself [n][hkv][dh]) into a cache
// [hkv][cap][dh] of the activation type at positions pos0 + t.
hipError_t launch_kv_append(const float* kself, const float* vself, int n, int hkv, int dh,
                            void* kc, void* vc, int cap, int pos0, int act, hipStream_t s);
hipError_t launch_qkv(const QkvArgs& a, int act, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int act, int n_work, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int act, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_init(const InitArgs& a, hipStream_t s);
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);

// Static device scratch (scratch.hip): STATIC_SCRATCH_BYTES in one file-scope __device__ array
// per GPU.  resolve_static_scratch takes its device address once per device (call with that
// device current); static_scratch returns it (nullptr until resolved).
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)64 << 20;
hipError_t resolve_static_scratch(int device);
void* static_scratch(int device);

// rows of Q per attention workgroup for the given activation type / head size
int attention_qblock(int act, int dh);
// attention workgroups resident per compute unit (LDS / register limited)
int attention_wgs_per_cu(int act, int dh);

}  // namespace ks
