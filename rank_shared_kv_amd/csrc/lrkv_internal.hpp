// Internal launch interface between the C ABI (lrkv_api.cpp) and the kernel
// translation units.  Every launcher only enqueues; arguments have already
// been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lrkv {

struct DecodeArgs {
    int batch, H, d_h, r, L_cap, dtype;
    int max_len;         // host bound of seq_lens
    int chunk;           // split granule in rows: split s holds live rows iff s * chunk < L_b
    int num_splits;      // G: workgroups of the launch = partial records per head (shared by the batch)
    int qgroup;          // virtual sequences per cached sequence: sequence b reads cache sequence b / qgroup
                         // (multi-token decode: one virtual sequence per set of qw query tokens, with the causal
                         // length of the set's last token)
    int n_queries;       // multi-token decode: query tokens per cached sequence (q and p rows [batch][n_queries][H])
    int qw;              // query tokens per virtual sequence: 1, or 2 / 4 for the bf16 matrix-core kernel, which
                         // then writes qw records per workgroup and head ([G][qw][H][record])
    const void* k_shared;
    const void* v_shared;
    const void* z_k;
    const void* z_v;
    const int32_t* seq_lens;
    const void* q;
    const float* p;
    const void* rho;     // normalised variant: scales [batch][L_cap][H] (cache dtype) multiplying the logits; else NULL
    float* ws;           // [G][H][record]
    // paged cache (block_table set): the four cache pointers are page pools [n_pages][page_rows][...] and
    // logical row t of sequence b is pool row block_table[b * max_pages + (t >> page_shift)] * page_rows
    // + (t & (page_rows - 1)); block_table NULL: contiguous [batch][L_cap][...]
    const int32_t* block_table;
    int page_shift, max_pages, n_pages;
    // rotary variant (rope_cs set): every key k_s + z^K_h (B^K_h)^T is turned at its row position and the query
    // at position L_b - 1; rope_cs holds (cos, sin) per position and coordinate pair [L_cap][d_h / 2][2], rope_bk
    // is B^K [H][d_h][r]; p is not used
    const float* rope_cs;
    const void* rope_bk;
    // fused decode step (lrkv_decode_step): one launch of n_absorb absorb workgroups (p = q B^K, four (b, h) units
    // each, written to p_out, which p also points at), the num_splits split workgroups and n_merge merge
    // workgroups (one per (b, h), writing out), handing work on through the counters at sync; every sequence is
    // seen at its appended length (append_cap = L_cap: the new token's rows k_new, v_new, zk_new, zv_new are
    // written at row seq_lens[b] when it is below L_cap, and the lengths grow at the end).  append_cap = 0 and
    // n_absorb = n_merge = 0 otherwise.
    int append_cap, n_absorb, n_merge, merge_wide;
    const void* k_new;
    const void* v_new;
    const void* zk_new;
    const void* zv_new;
    const void* B_k;
    const void* B_v;
    float* p_out;
    float* out;
    uint32_t* sync;
    int32_t* seq_lens_rw;  // the same lengths as seq_lens, grown by the last workgroup
};

// pool row of logical row t of sequence b (t uniform across the caller's wave)
__device__ __forceinline__ int paged_row(const DecodeArgs& a, int b, int t) {
    if (!a.block_table) return t;
    return (a.block_table[(size_t)b * a.max_pages + (t >> a.page_shift)] << a.page_shift) + (t & ((1 << a.page_shift) - 1));
}

// Which split kernel a problem uses.
enum class SplitPath { kGeneral, kMfmaBf16, kMfmaF32, kRopeMfma };

// Decode split plan: pure host arithmetic (no device query), so workspace
// sizes are known without a GPU.
struct SplitPlan {
    SplitPath path;
    int chunk;       // split granule in rows (the kernel's tile: rows a split advances per step)
    int num_splits;  // G: workgroups for the whole batch, dealt to sequences by length on the device
    int occupancy;   // MFMA kernels: waves per SIMD they are compiled for (1 or 2)
};

bool mfma_path_supports(int H, int d_h, int r, int dtype, int L_cap);      // bf16 MFMA kernel
bool mfma_all_variants(int H, int d_h, int r);  // its normalised and several-query instances exist for the shape
bool mfma_f32_path_supports(int H, int d_h, int r, int dtype, int L_cap);  // fp32 MFMA kernel (r = 0)
int mfma_f32_rows_per_tile();  // rows one fp32 MFMA-kernel split advances per step
int mfma_rows_per_tile(int H);  // rows one MFMA-kernel workgroup advances per step
int mfma_max_query_width(int H, int d_h, int r);  // multi-token decode: query tokens per bf16 MFMA workgroup (2 or 4)
bool general_path_supports(int H, int d_h, int r);
bool rope_mfma_path_supports(int H, int d_h, int r, int dtype);  // rotary variant, bf16 matrix-core kernel
int rope_mfma_rows_per_tile();
int rope_mfma_workgroups();  // G of the rotary bf16 matrix-core kernel (one workgroup per CU)
hipError_t launch_split_rope_mfma(const DecodeArgs& a, hipStream_t stream);
size_t general_lds_bytes(int H, int d_h, int r, bool rope = false);

hipError_t launch_absorb(int batch, int H, int d_h, int r, int dtype, const void* q, const void* B_k, float* p,
                         hipStream_t stream);
hipError_t launch_append(int batch, int H, int d_h, int r, int L_cap, int dtype, void* k_shared, void* v_shared,
                         void* z_k, void* z_v, int32_t* seq_lens, const void* k_new, const void* v_new,
                         const void* zk_new, const void* zv_new, hipStream_t stream);
hipError_t launch_split_general(const DecodeArgs& a, hipStream_t stream);
// append and absorb in one launch (the absorb's 16-byte vector path: r > 0, r a multiple of 16 / element bytes,
// d_h <= 256); contiguous cache
bool append_absorb_supported(int H, int d_h, int r, int dtype);
hipError_t launch_append_absorb(int batch, int H, int d_h, int r, int L_cap, int dtype, void* k_shared,
                                void* v_shared, void* z_k, void* z_v, int32_t* seq_lens, const void* k_new,
                                const void* v_new, const void* zk_new, const void* zv_new, const void* q,
                                const void* B_k, float* p, hipStream_t stream);
hipError_t launch_split_mfma(const DecodeArgs& a, int occupancy, hipStream_t stream);  // occupancy: waves per SIMD (1 or 2)
// fused decode step on the bf16 matrix-core kernel (single query, contiguous cache); a carries the step fields
hipError_t launch_step_mfma(const DecodeArgs& a, int occupancy, hipStream_t stream);
bool merge_wide(int num_splits, int n_virtual);  // the merge's split grouping (4 groups when true)
hipError_t launch_split_mfma_f32(const DecodeArgs& a, int occupancy, hipStream_t stream);
// decode step's split pass on the fp32 rank-0 matrix-core kernel: a carries the step fields (the pass appends the
// token and its last workgroup grows the lengths); the merge kernel runs after it on the grown lengths
hipError_t launch_step_mfma_f32(const DecodeArgs& a, int occupancy, hipStream_t stream);
// Merge of a decode of `batch` cached sequences with Q query tokens each, split as virtual sequences of qw
// tokens (ceil(Q / qw) per cached sequence; seq_lens are their lengths, num_splits the split launch's G);
// out [batch][Q][H][d_h].  Single-token decode: Q = qw = 1.
hipError_t launch_merge(int batch, int Q, int qw, int H, int d_h, int r, int dtype, int max_len, int chunk,
                        int num_splits, const int32_t* seq_lens, const void* B_v, float* out, const float* ws,
                        hipStream_t stream);
// the split plan of a single-query launch (append_cap: 0, or L_cap for the fused step): W_b and S_b per sequence
hipError_t launch_split_plan(int batch, int max_len, int append_cap, int chunk, int num_splits,
                             const int32_t* seq_lens, int32_t* first_wg, int32_t* splits, hipStream_t stream);
int general_rows_per_tile();  // rows one general-kernel split advances per step
hipError_t launch_project_append(int batch, int H, int d_h, int r, int L_cap, int dtype, int d_model, void* k_shared,
                                 void* v_shared, void* z_k, void* z_v, int32_t* seq_lens, const void* x,
                                 const void* W_in, void* q_out, hipStream_t stream);
hipError_t launch_materialize(int batch, int H, int d_h, int r, int L_cap, int dtype, int max_len,
                              const int32_t* seq_lens, const void* k_shared, const void* v_shared, const void* z_k,
                              const void* z_v, const void* B_k, const void* B_v, void* K_out, void* V_out,
                              hipStream_t stream);
// Virtual lengths of a multi-token decode split into sets of qw tokens: lens_out[b * nc + c] (nc = ceil(Q / qw))
// is the number of rows the last token of set c of sequence b sees, max(0, seq_lens[b] - Q + 1 + last) with
// last = min((c + 1) * qw, Q) - 1 (token i sees seq_lens[b] - Q + 1 + i rows)
hipError_t launch_multi_lengths(int batch, int Q, int qw, const int32_t* seq_lens, int32_t* lens_out,
                                hipStream_t stream);
hipError_t launch_paged_append(int batch, int H, int d_h, int r, int dtype, int page_shift, int max_pages,
                              void* k_pages, void* v_pages, void* zk_pages, void* zv_pages,
                              const int32_t* block_table, int32_t* seq_lens, const void* k_new, const void* v_new,
                              const void* zk_new, const void* zv_new, hipStream_t stream);
// latents from the per-head layout [batch][H][L_cap][r] to the token-major one [batch][L_cap][H][r]
hipError_t launch_latents_token_major(int batch, int H, int L_cap, int r, int dtype, const void* src, void* dst,
                                      hipStream_t stream);
int read_probe_workgroups();
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_rope_table(int d_h, int n_pos, float base, float* table, hipStream_t stream);
hipError_t launch_key_scales(int batch, int H, int d_h, int r, int L_cap, int dtype, int max_len, int n_last,
                             float eps, const int32_t* seq_lens, const void* k_shared, const void* z_k,
                             const void* B_k, void* rho, hipStream_t stream);
hipError_t launch_norm_query(int batch, int H, int d_h, int dtype, float eps, const void* q, const void* g_q,
                             const void* g_k, void* q_eff, hipStream_t stream);
hipError_t launch_output_project(int batch, int H, int d_h, int dtype, int d_model, const float* o, const void* W_o,
                                 float* y, hipStream_t stream);

}  // namespace lrkv
