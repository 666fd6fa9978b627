// la_internal.h -- host-side plan and launcher interface shared by the C ABI
// (la_abi.cpp) and the kernel translation units.  No HIP types here.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace la {

// How a forward pass is laid out.  A "chunk" is a run of C tokens of one
// sequence (C a multiple of the block size) that one workgroup walks block by
// block, carrying the d x d state.  The state at each chunk's start comes
// from a parallel segmented exclusive scan over the K^T V summaries of
// "sub-chunks" of C_s tokens (C a multiple of C_s): chunks are sized to fill
// the chip, sub-chunks to give the summary kernel enough workgroups.
struct FwdPlan {
    int64_t chunk = 0;        // C, tokens per chunk
    int64_t sub = 0;          // C_s, tokens per sub-chunk
    int scan_group = 0;       // G, sub-chunks per scan tile
    int64_t nchunk_ub = 0;    // chunk slots per head (exact for dense input)
    int64_t nsub_ub = 0;      // sub-chunk slots per head
    int64_t ntile_ub = 0;     // scan-tile slots per head
    bool scan_tiles = false;  // some sequence may span more than G sub-chunks
    bool single_chunk = false;  // every sequence is one chunk: no summaries, no scan
    size_t off_chunk_off = 0; // int32 [nseq + 1]
    size_t off_sub_off = 0;   // int32 [nseq + 1]
    size_t off_err = 0;       // int32: 1 when cu_seqlens was found malformed (packed input)
    size_t off_perm = 0;      // int32 [nseq] (packed input: sequences longest first)
    size_t off_rank_off = 0;  // int32 [nseq + 1]
    size_t off_slot_tab = 0;  // int32 [nchunk_ub][2] (packed input: sequence and chunk of each chunk slot)
    size_t off_tile_off = 0;  // int32 [nseq + 1]
    size_t off_states = 0;    // fp32 [heads][nsub_ub][d][d]
    size_t off_tilesum = 0;   // fp32 [heads][ntile_ub][d][d]
    size_t bytes = 0;         // total workspace bytes
};

// Argument checks shared by the size query and the forward call.  Returns an
// LA_* status (LA_OK when the shape is supported).
int check_fwd_shape(int batch, int heads, int64_t seq_len, int head_dim, int block_size,
                    int dtype);

// Chunk and sub-chunk lengths given by the caller instead of chosen by the
// planner (0 = the planner's choice).  Only the test entry point
// lightning_attn_fwd_planned sets them; nothing reads them from the
// environment.
struct PlanOverride {
    int64_t chunk = 0;
    int64_t sub = 0;
};

// Fill *plan for a checked shape (seq_len > 0) on a device with `cus`
// compute units.  Returns LA_OK, or LA_EINVAL when an override is not a
// valid chunk / sub-chunk length for the shape (then *plan is untouched).
int make_fwd_plan(int batch, int heads, int64_t seq_len, int head_dim, int block_size,
                  bool varlen, int cus, const PlanOverride &ov, FwdPlan *plan);

// Compute units of the current HIP device, read once per device from its
// properties and cached (256 when no device can be queried, e.g. a host
// without a GPU).
int device_cu_count();

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    int nseq, heads, head_dim, block_size, dtype;
    int64_t seq_len;          // dense: tokens per sequence; packed: total tokens
    const int32_t *cu_seqlens;  // device, or nullptr for dense input
    const float *s_init;      // device [nseq][heads][d][d] or nullptr (zero)
    float *s_final;           // device [nseq][heads][d][d] or nullptr (not wanted)
    const int32_t *slots = nullptr;  // device [nseq]: with it s_init == s_final is a pool
    int nslots = 0;                  // of nslots entries; sequence s uses entry slots[s]
    int rope_dims = 0;        // > 0: rotate the first rope_dims dims of q and k (bf16)
    double rope_base = 0.0;   // rotary base frequency
    const int32_t *pos0 = nullptr;  // device [nseq]: position of each first token, or nullptr (0)
    char *workspace;
    FwdPlan plan;
};

// Queue the forward kernels on `stream` (a hipStream_t).  When `events` is
// non-null it holds 5 hipEvent_t handles recorded at the stage boundaries.
// Returns 0 or a HIP error code.
int launch_fwd(const FwdArgs &a, void *stream, void *const *events);

// Wait for `stream` and read the flag k_prep raises for a malformed
// cu_seqlens (packed input).  Returns 0 or a HIP error code.
int read_cu_error(const FwdArgs &a, void *stream, int *flag);

// Queue the kernel that sets the final state of every sequence of length 0
// (all of them when there are no tokens at all) to its initial state.
int launch_state_empty(const float *s_init, float *s_final, int nseq, int heads, int head_dim,
                       void *stream);

// Queue one decode step.  With `slots` non-null, row b's state is entry
// slots[b] of a pool of `nslots` (out-of-range slots are padding rows).
// Returns 0 or a HIP error code.
int launch_decode(const void *q, const void *k, const void *v, float *state, void *o,
                  int batch, int heads, int head_dim, int dtype, void *stream,
                  const int32_t *slots = nullptr, int nslots = 0, int rope_dims = 0,
                  double rope_base = 0.0, const int32_t *positions = nullptr);

}  // namespace la
