// Host-side interface between the C ABI (api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tka {

struct ScoreArgs {
  const void* q;     // [B,Hq,d]
  const void* keys;  // rows of d elements at b*sb + g*sh + i*sl
  float* scores;     // [B,Hq,nrows]
  int B, Hq, Hkv, G, d, nrows;
  int64_t sb, sh, sl;
  float scale;
  int bf16;    // rows: 1 bf16, 0 fp32
  int q_bf16;  // query: 1 bf16, 0 fp32
  int M = 1;   // queries per sequence (q [B,M,Hq,d], scores [B,M,Hq,nrows], causal)
  int block = 0;  // rows are fp32 block means (one query per sequence)
  uint32_t* rmax = nullptr;  // optional: partial row maxima (score keys), score_rmax_slots per row
};

struct IndexerArgs {
  const uint8_t* qI;  // [B,HI,dI]
  const uint8_t* kI;  // [B,Lc,dI]
  const float* w;     // [B,HI]
  float* scores;      // [B,L]
  int B, HI, dI, L;
  int Lc;             // positions per sequence in kI (>= L)
};

struct HisaArgs {
  const void* q;      // [B,Hq,d]
  const void* K;      // strided cache
  const int32_t* blk; // [B*Hq, KB] kept blocks, ascending, -1 padded
  float* cand;        // [B*Hq, KB*bsz]
  int32_t* krow;      // [B*Hq]
  int B, Hq, G, d, L, KB, bsz, k;
  int64_t sb, sh, sl;
  float scale;
  int bf16;
};

struct BlockMeanArgs {
  const void* K;
  float* means;  // [B,Hkv,m,d]
  int B, Hkv, d, L, bsz, m;
  int64_t sb, sh, sl;
  int bf16;
  int j0 = 0, j1 = 0;  // blocks [j0, j1) only (j1 = 0: all m)
};

struct SelectArgs {
  const float* scores;
  int64_t n_rows;
  int n;  // row length
  int64_t stride;
  int k;
  int32_t* idx;
  float* sel;  // nullable
};

struct GatherArgs {
  const void* q;
  const void* K;
  const void* V;
  const int32_t* idx;
  const float* sel;  // nullable
  float* out;
  int B, Hq, Hkv, G, d, L;
  int64_t sb, sh, sl;
  float scale;
  int bf16;
  int n_idx, unit, shared;
  int M = 1;  // queries per sequence: B counts (sequence, query) pairs, K/V rows are those of B / M
};

// Outputs of the exact bf16 MFMA scan (see score.hip for the modes).
struct MfmaOut {
  float* S;                     // full scores [B*Hq, L], or sample scores [B*Hq, nsamp]
  int nsamp;
  const float* T;               // candidate scan: score threshold per row (kept: ranks >= T)
  uint32_t* cnt;                // candidate mode: candidates found per row
  uint32_t* cbits;              // candidate mode: [B*Hq, capg] score bits
  int32_t* cpos;                // candidate mode: [B*Hq, capg] positions
  uint2* cpair;                 // candidate mode, packed (when set, instead of cbits/cpos): [B*Hq, capg] (bits, pos)
  int capg;
  int stage;                    // candidate mode: LDS staging entries per head
  uint32_t* rmax;               // full mode, optional: [B*Hq, rmax_slots] maxima of score keys, one per
  int rmax_slots;               //   (workgroup chunk, wave) of the row
};

// Largest LDS a workgroup may take on the current device, and a one-time
// (per kernel and device) permission for a kernel to use more than 64 KiB.
int device_lds_limit();
void ensure_dynamic_lds(const void* kernel, size_t bytes);

bool score_uses_mfma(int dtype_bf16, int G);
int mfma_scan_chunk(const ScoreArgs& a);
void launch_score_mfma_sample(const ScoreArgs& a, int sample_chunk, int nsamp, float* samp, hipStream_t st);
void launch_score_mfma_cand(const ScoreArgs& a, const MfmaOut& o, hipStream_t st);
void launch_score_dense(const ScoreArgs& a, hipStream_t st);
// Partial row maxima the dense scores can write beside the scores (ScoreArgs.rmax): the number
// per row, 0 where the launch writes none (then rmax is ignored).
int score_rmax_slots(const ScoreArgs& a);
void launch_score_indexer(const IndexerArgs& a, hipStream_t st);
void launch_block_mean(const BlockMeanArgs& a, hipStream_t st);
// append one position of every (b, KV head) row (16-byte rows) and/or encode indexer keys
void launch_append_rows(const void* knew, const void* vnew, void* K, void* V, int B, int Hkv, int row_bytes, int es,
                        int64_t sb, int64_t sh, int64_t sl, int pos, hipStream_t st);
void launch_append_indexer(const float* kI_new, uint8_t* kI, int B, int dI, int Lc, int pos, hipStream_t st);

size_t select_workspace_bytes(int64_t n_rows, int n, int k);
bool select_len_supported(int64_t n_rows, int n);  // false: rows too long for the split finish
void launch_select(const SelectArgs& a, void* ws, hipStream_t st);
// one workgroup per row, only rows whose flag is nonzero
// certified adaptive k per row (a.k = k_max): counts to kout and the kept positions, then
// tau; W, M and row_flag [n_rows] are scratch
// rmax (optional, rslots per row): partial maxima of each row's score keys that the scoring pass
// wrote (ScoreArgs.rmax); the long-row path then skips its pass for the row maximum.
void launch_select_adaptive(const SelectArgs& a, float eps, int k_min, int32_t* kout, uint64_t* W, float* M,
                            uint32_t* row_flag, float* tau, hipStream_t st, const uint32_t* rmax = nullptr,
                            int rslots = 0);
// several causal queries per sequence: exact scores (bf16, M*G <= 64 rows per KV head; a
// position a query cannot see is NaN) and each row's count min(k, L - M + t + 1)
void launch_score_mq(const ScoreArgs& a, hipStream_t st);
void launch_mq_counts(int32_t* krow, int64_t rows, int M, int Hq, int L, int k, hipStream_t st);
// the two-level step's fine level: token scores of the kept blocks, and slot -> position
void launch_hisa_token_scores(const HisaArgs& a, hipStream_t st);
void launch_hisa_map(int32_t* idx, const int32_t* blk, int64_t rows, int k, int KB, int bsz, hipStream_t st);
// row select with a count per row (krow[r] <= a.k; rows padded with -1 up to a.k)
void launch_select_rows_counts(const SelectArgs& a, const int32_t* krow, hipStream_t st);
// rows with row_flag set; krow (optional): each row's count, at most a.k
void launch_select_rows_flagged(const SelectArgs& a, const uint32_t* row_flag, const int32_t* krow, hipStream_t st);

// candidate prefilter of the fused exact step (select.hip)
void launch_prefilter_threshold(const float* samp, int64_t n_rows, int nsamp, int r, float* T, uint32_t* cnt,
                                uint32_t* row_flag, uint32_t* group_flag, int G, int Hq, int M, hipStream_t st);
// rows are (b, t, h) with M queries t per sequence; group flags are per (b, KV head)
void launch_prefilter_finish(const uint2* cpair, const uint32_t* cnt, const float* T,
                             int capg, int64_t n_rows, int n, int k, int G, int Hq, int M, int32_t* idx, float* sel,
                             uint32_t* row_flag, uint32_t* group_flag, hipStream_t st);

// repair of the rows the prefilter flagged: exact scores of their groups' 16-row blocks into
// bounded slots (repair_slot_bytes), then the row select of each flagged row
// The indexer variant's fused select: each scoring workgroup keeps its chunk's first positions in the
// select order as candidates; one workgroup per sequence selects among them (or, when a chunk could
// hold more kept positions than it kept, over the whole score row).
struct IndexerCandPlan {
  bool on = false;
  int nch = 0;    // chunks per sequence
  int ncand = 0;  // candidates per sequence
};
IndexerCandPlan indexer_cand_plan(int L, int k);
size_t indexer_cand_bytes(int64_t B, const IndexerCandPlan& pl);
// scores (a.scores, [B, L]) and candidates, then idx [B, k] ascending (-1 padded) and sel (optional)
void launch_indexer_select(const IndexerArgs& a, const IndexerCandPlan& pl, int k, void* cand_ws, int32_t* idx,
                           float* sel, hipStream_t st);

struct RepairArgs {
  const void* q;
  const void* K;
  int B, Hq, Hkv, G, M, d, L, k;
  int64_t sb, sh, sl;
  float scale;
  const uint32_t* group_flag;
  const uint32_t* row_flag;
  float* slots;
  int32_t* idx;
  float* sel;
};
size_t repair_slot_bytes(int64_t n_groups, int rows_per_group, int L);
void launch_prefilter_repair(const RepairArgs& a, hipStream_t st);

// gather planning is shared by the workspace query and the launch
struct GatherPlan {
  int tasks, heads_per_task, span, nsplit;
  int64_t expanded;  // tokens per task after block expansion
  size_t ws_bytes;
};
GatherPlan plan_gather(const GatherArgs& a);
void launch_gather(const GatherArgs& a, const GatherPlan& pl, void* ws, hipStream_t st);

}  // namespace tka
