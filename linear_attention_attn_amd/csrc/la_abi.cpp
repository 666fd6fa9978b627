// la_abi.cpp -- the extern "C" entry points of liblightning_attn.so.
//
// Validation, workspace planning and dispatch.  Every check runs on the host
// before any HIP call, so a rejected call has no side effects.  The library
// allocates nothing: the caller passes all device memory, including the
// workspace sized by lightning_attn_fwd_workspace_size.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>

#include "../../include/lightning_attn.h"
#include "la_internal.h"

namespace la {

static bool dtype_ok(int dtype) { return dtype == LA_DTYPE_BF16 || dtype == LA_DTYPE_F32; }

int check_fwd_shape(int batch, int heads, int64_t seq_len, int head_dim, int block_size, int dtype) {
    if (!dtype_ok(dtype)) return LA_EUNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return LA_EUNSUPPORTED;
    if (block_size != 64 && block_size != 128 && block_size != 256) return LA_EUNSUPPORTED;
    if (batch < 1 || heads < 1 || seq_len < 0) return LA_EINVAL;
    if (heads > 65535) return LA_EUNSUPPORTED;          // heads run along grid y
    if (seq_len > (int64_t)INT32_MAX) return LA_EUNSUPPORTED;  // int32 cu_seqlens / tables
    return LA_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The kernels move q, k, v, o and states in 16-byte vectors.
static bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }
// int32 tables (cu_seqlens, slots, positions, offsets).
static bool aligned4(const void *p) { return ((uintptr_t)p & 3) == 0; }

// The decode step runs one 256-thread workgroup per (row, head): at most
// 2^32 - 1 work-items in one launch.
static bool decode_grid_ok(int batch, int heads) {
    return (int64_t)batch * heads * 256 <= ((int64_t)1 << 32) - 1;
}

static int64_t env_i64(const char *name, int64_t dflt) {
    const char *s = getenv(name);
    if (!s || !*s) return dflt;
    char *end = nullptr;
    long long v = strtoll(s, &end, 10);
    return (end && *end == 0 && v > 0) ? (int64_t)v : dflt;
}

// Chunk length C (tokens one workgroup walks carrying the state; a multiple
// of the block size) and sub-chunk length C_s (the K^T V summary granularity;
// C is a multiple of C_s, C_s <= kSub).
//
// Dense input: every candidate C is priced with a simple model of the two
// passes in units of "tokens one CU streams through the fused kernel":
//   fused   = ceil(units * n / cus) * C      (rounds of one chunk per CU)
//   summary = kSum * units * (n - 1) * C / cus   (every chunk but the last is
//             summarised; measured ~0.45 of the fused cost per token)
//   scan    = kScan * units * n_s / cus      (three passes over 64 KiB fp32
//             states per sub-chunk, ~190 token-equivalents each)
// with n = ceil(L / C) chunks and n_s = ceil(L / C_s) sub-chunks per unit.
// Candidates: one chunk per sequence (no summary or scan at all), powers of
// two from the block size to kSub, and multiples of kSub (sub-chunks of kSub),
// all within the 32-bit buffer offsets of the bf16 kernels (2^30 bytes of a
// chunk's rows).  E.g. 64 heads x 1M tokens on 256 CUs: C = 262144 (4 chunks
// per head, one workgroup per CU) with sub-chunks of 16384, so the summaries
// read 3/4 of k and v instead of 63/64 with 16384-token chunks.
//
// Packed input (the lengths live on the device): C = the largest power of
// two <= W / cus (W = all head-tokens), so that there are at least about
// cus chunks and no chunk is longer than a CU's average share; sub-chunks of
// at most kSub.  The fused kernel takes the chunks of the longest sequences
// first, so the long ones do not start last.
//
// An override (test entry point only) fixes C: a multiple of the block size
// within the offset cap, and above kSub a multiple of kSub; and C_s: a
// multiple of the block size dividing C (ignored when one chunk covers every
// dense sequence).  Anything else is LA_EINVAL.
int make_fwd_plan(int batch, int heads, int64_t seq_len, int head_dim, int block_size, bool varlen,
                  int cus, const PlanOverride &ov, FwdPlan *plan) {
    const int64_t kCUs = cus > 0 ? cus : 256;
    const int64_t kSub = 16384;
    const double kSum = 0.45, kScan = 190.0;
    const int64_t units = (int64_t)batch * heads;
    const int64_t B = block_size;
    const int64_t cap = (((int64_t)1 << 30) / (head_dim * 2)) / B * B;
    auto cdiv = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
    if (ov.chunk < 0 || ov.sub < 0) return LA_EINVAL;

    int64_t C;
    if (ov.chunk > 0) {
        if (ov.chunk % B != 0 || ov.chunk > cap || (ov.chunk > kSub && ov.chunk % kSub != 0))
            return LA_EINVAL;
        C = ov.chunk;
    } else if (!varlen) {
        const int64_t L = std::max<int64_t>(1, seq_len);
        auto cost = [&](int64_t c) {
            const int64_t n = cdiv(L, c);
            const int64_t cs = n == 1 ? c : std::min(c, kSub);
            const double fused = (double)cdiv(units * n, kCUs) * (double)std::min(c, L);
            const double summ = kSum * (double)units * (double)(n - 1) * (double)c / (double)kCUs;
            const double scan = n == 1 ? 0.0 : kScan * (double)units * (double)cdiv(L, cs) / (double)kCUs;
            return fused + summ + scan;
        };
        C = B;
        double best = cost(C);
        auto consider = [&](int64_t c) {
            if (c < B || c > cap || c % B) return;
            const double v = cost(c);
            if (v < best) { best = v; C = c; }       // ties keep the smaller chunk
        };
        for (int64_t c = B; c <= kSub; c *= 2) consider(c);
        for (int64_t m = 2; m * kSub < L + kSub && m * kSub <= cap; ++m) consider(m * kSub);
        consider(cdiv(L, B) * B);                     // one chunk per sequence
    } else {
        const int64_t lavg = std::max<int64_t>(1, seq_len / batch);
        const int64_t per_cu = std::max<int64_t>(1, units * lavg / kCUs);
        C = B;
        while (C * 2 <= cap && C * 2 <= per_cu) C *= 2;
    }
    const bool one = !varlen && cdiv(std::max<int64_t>(1, seq_len), C) == 1;
    int64_t Cs = one ? C : std::min(C, kSub);
    if (ov.sub > 0 && !one) {
        if (ov.sub % B != 0 || C % ov.sub != 0) return LA_EINVAL;
        Cs = ov.sub;
    }

    const int G = 32;
    FwdPlan p;
    p.chunk = C;
    p.sub = Cs;
    p.scan_group = G;
    if (!varlen) {
        const int64_t cps = cdiv(seq_len, C), sps = cdiv(seq_len, Cs);
        p.nchunk_ub = (int64_t)batch * cps;
        p.nsub_ub = (int64_t)batch * sps;
        p.ntile_ub = (int64_t)batch * cdiv(sps, G);
        p.scan_tiles = sps > G;
        p.single_chunk = cps == 1;
    } else {
        p.nchunk_ub = seq_len / C + batch;
        // Only a sequence longer than C has sub-chunk entries, (nc - 1) C / Cs + 1
        // < L / Cs + 1 of them, and there are at most T / C such sequences.
        p.nsub_ub = seq_len / Cs + seq_len / C;
        p.ntile_ub = p.nsub_ub / G + 1 + seq_len / C;
        p.scan_tiles = cdiv(seq_len, Cs) > G;
        p.single_chunk = seq_len <= C;   // no sequence is longer than the whole input
    }
    // One launch covers at most 2^32 - 1 work-items along x: the fused
    // kernels run up to 1024 threads per chunk, the summaries 512 per
    // sub-chunk, the scan and empty-state kernels 256 per tile or sequence.
    const int64_t kMaxX = ((int64_t)1 << 32) - 1;
    if (p.nchunk_ub * 1024 > kMaxX || (int64_t)batch * 256 > kMaxX) return LA_EUNSUPPORTED;
    if (!p.single_chunk && (p.nsub_ub * 512 > kMaxX || p.ntile_ub * 256 > kMaxX)) return LA_EUNSUPPORTED;
    const size_t dd = (size_t)head_dim * head_dim * sizeof(float);
    size_t off = 0;
    p.off_chunk_off = off;
    off = align256(off + (size_t)(batch + 1) * sizeof(int32_t));
    p.off_sub_off = off;
    off = align256(off + (size_t)(batch + 1) * sizeof(int32_t));
    if (varlen) {
        p.off_err = off;
        off = align256(off + sizeof(int32_t));
        p.off_perm = off;
        off = align256(off + (size_t)batch * sizeof(int32_t));
        p.off_rank_off = off;
        off = align256(off + (size_t)(batch + 1) * sizeof(int32_t));
        p.off_slot_tab = off;
        off = align256(off + (size_t)p.nchunk_ub * 2 * sizeof(int32_t));
    }
    p.off_tile_off = off;
    off = align256(off + (size_t)(batch + 1) * sizeof(int32_t));
    p.off_states = off;
    off = align256(off + (size_t)heads * (size_t)p.nsub_ub * dd);
    p.off_tilesum = off;
    if (p.scan_tiles) off = align256(off + (size_t)heads * (size_t)p.ntile_ub * dd);
    p.bytes = off;
    *plan = p;
    return LA_OK;
}

}  // namespace la

extern "C" {

size_t lightning_attn_fwd_workspace_size(int batch, int heads, int64_t seq_len, int head_dim,
                                         int block_size, int varlen, int dtype) {
    return lightning_attn_fwd_workspace_size_planned(batch, heads, seq_len, head_dim, block_size, varlen,
                                                     dtype, 0, 0);
}

size_t lightning_attn_fwd_workspace_size_planned(int batch, int heads, int64_t seq_len, int head_dim,
                                                 int block_size, int varlen, int dtype,
                                                 int64_t chunk_tokens, int64_t sub_tokens) {
    if (la::check_fwd_shape(batch, heads, seq_len, head_dim, block_size, dtype) != LA_OK) return 0;
    if (seq_len == 0) return 0;
    la::FwdPlan p;
    la::PlanOverride ov;
    ov.chunk = chunk_tokens;
    ov.sub = sub_tokens;
    if (la::make_fwd_plan(batch, heads, seq_len, head_dim, block_size, varlen != 0, la::device_cu_count(),
                          ov, &p) != LA_OK)
        return 0;
    return p.bytes;
}

int64_t lightning_attn_fwd_chunk_tokens(int batch, int heads, int64_t seq_len, int head_dim,
                                        int block_size, int varlen, int dtype) {
    if (la::check_fwd_shape(batch, heads, seq_len, head_dim, block_size, dtype) != LA_OK) return 0;
    if (seq_len == 0) return 0;
    la::FwdPlan p;
    la::make_fwd_plan(batch, heads, seq_len, head_dim, block_size, varlen != 0, la::device_cu_count(),
                      la::PlanOverride{}, &p);
    return p.chunk;
}

// Rotary arguments: rope_dims 0 (none) or head_dim / 2 with a finite base > 0.
static int check_rope(int rope_dims, double rope_base, int head_dim) {
    if (rope_dims == 0) return LA_OK;
    if (rope_dims != head_dim / 2) return LA_EUNSUPPORTED;
    if (!(rope_base > 0.0) || !isfinite(rope_base)) return LA_EINVAL;
    return LA_OK;
}

static int fwd_common(const void *q, const void *k, const void *v, void *o, int batch, int heads,
                      int64_t seq_len, int head_dim, int block_size, const int32_t *cu_seqlens,
                      int dtype, const float *s_init, float *s_final, void *workspace,
                      size_t workspace_bytes, void *stream, void *const *events,
                      int rope_dims = 0, double rope_base = 0.0, const int32_t *pos0 = nullptr,
                      const int32_t *slots = nullptr, int nslots = 0,
                      la::PlanOverride ov = la::PlanOverride{}) {
    int st = la::check_fwd_shape(batch, heads, seq_len, head_dim, block_size, dtype);
    if (st != LA_OK) return st;
    st = check_rope(rope_dims, rope_base, head_dim);
    if (st != LA_OK) return st;
    if (((uintptr_t)s_init & 15) != 0 || ((uintptr_t)s_final & 15) != 0) return LA_EINVAL;
    if (seq_len == 0) {
        // no tokens: only the final states (each equal to its initial state;
        // a pool entry is updated in place, so there is nothing to do)
        if (!s_final || slots) return LA_OK;
        return la::launch_state_empty(s_init, s_final, batch, heads, head_dim, stream) == 0 ? LA_OK : LA_EHIP;
    }
    if (!q || !k || !v || !o) return LA_EINVAL;
    if (!la::aligned16(q) || !la::aligned16(k) || !la::aligned16(v) || !la::aligned16(o)) return LA_EINVAL;
    if (!la::aligned4(cu_seqlens) || !la::aligned4(pos0) || !la::aligned4(slots)) return LA_EINVAL;
    la::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.nseq = batch; a.heads = heads; a.head_dim = head_dim; a.block_size = block_size;
    a.dtype = dtype; a.seq_len = seq_len; a.cu_seqlens = cu_seqlens;
    a.s_init = s_init; a.s_final = s_final;
    a.rope_dims = rope_dims; a.rope_base = rope_base; a.pos0 = pos0;
    a.slots = slots; a.nslots = nslots;
    st = la::make_fwd_plan(batch, heads, seq_len, head_dim, block_size, cu_seqlens != nullptr,
                           la::device_cu_count(), ov, &a.plan);
    if (st != LA_OK) return st;
    if (!workspace || workspace_bytes < a.plan.bytes) return LA_EWORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return LA_EINVAL;
    a.workspace = static_cast<char *>(workspace);
    if (la::launch_fwd(a, stream, events) != 0) return LA_EHIP;
    if (cu_seqlens && la::env_i64("LA_DEBUG_CHECKS", 0) > 0) {
        int bad = 0;
        if (la::read_cu_error(a, stream, &bad) != 0) return LA_EHIP;
        if (bad) return LA_EINVAL;
    }
    return LA_OK;
}

int lightning_attn_fwd(const void *q, const void *k, const void *v, void *o, int batch, int heads,
                       int64_t seq_len, int head_dim, int block_size, const int32_t *cu_seqlens,
                       int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return fwd_common(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens, dtype,
                      nullptr, nullptr, workspace, workspace_bytes, stream, nullptr);
}

int lightning_attn_fwd_state(const void *q, const void *k, const void *v, void *o, int batch,
                             int heads, int64_t seq_len, int head_dim, int block_size,
                             const int32_t *cu_seqlens, int dtype, const float *s_init,
                             float *s_final, void *workspace, size_t workspace_bytes,
                             void *stream) {
    return fwd_common(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens, dtype,
                      s_init, s_final, workspace, workspace_bytes, stream, nullptr);
}

int lightning_attn_fwd_rope(const void *q, const void *k, const void *v, void *o, int batch,
                            int heads, int64_t seq_len, int head_dim, int block_size,
                            const int32_t *cu_seqlens, int dtype, int rope_dims, double rope_base,
                            const int32_t *pos_offset, const float *s_init, float *s_final,
                            void *workspace, size_t workspace_bytes, void *stream) {
    if (rope_dims <= 0) return LA_EUNSUPPORTED;
    return fwd_common(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens, dtype,
                      s_init, s_final, workspace, workspace_bytes, stream, nullptr, rope_dims,
                      rope_base, pos_offset);
}

int lightning_attn_fwd_indexed(const void *q, const void *k, const void *v, void *o, int batch,
                               int heads, int64_t seq_len, int head_dim, int block_size,
                               const int32_t *cu_seqlens, int dtype, float *state_pool, int nslots,
                               const int32_t *slots, int rope_dims, double rope_base,
                               const int32_t *pos_offset, void *workspace, size_t workspace_bytes,
                               void *stream) {
    if (!slots || nslots < 0 || (nslots > 0 && !state_pool)) return LA_EINVAL;
    if ((int64_t)nslots * heads > (int64_t)INT32_MAX) return LA_EUNSUPPORTED;
    return fwd_common(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens, dtype,
                      state_pool, state_pool, workspace, workspace_bytes, stream, nullptr, rope_dims,
                      rope_base, pos_offset, slots, nslots);
}

int lightning_attn_fwd_planned(const void *q, const void *k, const void *v, void *o, int batch,
                               int heads, int64_t seq_len, int head_dim, int block_size,
                               const int32_t *cu_seqlens, int dtype, const float *s_init,
                               float *s_final, float *state_pool, int nslots, const int32_t *slots,
                               int rope_dims, double rope_base, const int32_t *pos_offset,
                               int64_t chunk_tokens, int64_t sub_tokens, void *workspace,
                               size_t workspace_bytes, void *stream) {
    la::PlanOverride ov;
    ov.chunk = chunk_tokens;
    ov.sub = sub_tokens;
    if (rope_dims < 0) return LA_EUNSUPPORTED;
    if (slots) {
        if (s_init || s_final || nslots < 0 || (nslots > 0 && !state_pool)) return LA_EINVAL;
        if ((int64_t)nslots * heads > (int64_t)INT32_MAX) return LA_EUNSUPPORTED;
        return fwd_common(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens, dtype,
                          state_pool, state_pool, workspace, workspace_bytes, stream, nullptr, rope_dims,
                          rope_base, pos_offset, slots, nslots, ov);
    }
    if (state_pool) return LA_EINVAL;
    return fwd_common(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens, dtype, s_init,
                      s_final, workspace, workspace_bytes, stream, nullptr, rope_dims, rope_base,
                      pos_offset, nullptr, 0, ov);
}

int lightning_attn_fwd_traced(const void *q, const void *k, const void *v, void *o, int batch,
                              int heads, int64_t seq_len, int head_dim, int block_size,
                              const int32_t *cu_seqlens, int dtype, void *workspace,
                              size_t workspace_bytes, void *stream, void *const *events,
                              int nevents) {
    if (!events || nevents != LA_FWD_NUM_EVENTS) return LA_EINVAL;
    return fwd_common(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens, dtype,
                      nullptr, nullptr, workspace, workspace_bytes, stream, events);
}

int lightning_attn_decode(const void *q, const void *k, const void *v, float *state, void *o, int batch,
                          int heads, int head_dim, int dtype, void *stream) {
    if (!(dtype == LA_DTYPE_BF16 || dtype == LA_DTYPE_F32)) return LA_EUNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return LA_EUNSUPPORTED;
    if (batch < 1 || heads < 1) return LA_EINVAL;
    if (!la::decode_grid_ok(batch, heads)) return LA_EUNSUPPORTED;
    if (!q || !k || !v || !state || !o) return LA_EINVAL;
    if (!la::aligned16(state)) return LA_EINVAL;
    return la::launch_decode(q, k, v, state, o, batch, heads, head_dim, dtype, stream) == 0 ? LA_OK : LA_EHIP;
}

int lightning_attn_decode_indexed(const void *q, const void *k, const void *v, float *state_pool,
                                  int nslots, const int32_t *slots, void *o, int batch, int heads,
                                  int head_dim, int dtype, void *stream) {
    if (!(dtype == LA_DTYPE_BF16 || dtype == LA_DTYPE_F32)) return LA_EUNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return LA_EUNSUPPORTED;
    if (batch < 1 || heads < 1 || nslots < 0) return LA_EINVAL;
    if (!la::decode_grid_ok(batch, heads) || (int64_t)nslots * heads > (int64_t)INT32_MAX)
        return LA_EUNSUPPORTED;
    if (!q || !k || !v || !slots || !o || (nslots > 0 && !state_pool)) return LA_EINVAL;
    if (!la::aligned16(state_pool) || !la::aligned4(slots)) return LA_EINVAL;
    return la::launch_decode(q, k, v, state_pool, o, batch, heads, head_dim, dtype, stream, slots,
                             nslots) == 0 ? LA_OK : LA_EHIP;
}

int lightning_attn_decode_rope(const void *q, const void *k, const void *v, float *state, int nslots,
                               const int32_t *slots, void *o, int batch, int heads, int head_dim,
                               int dtype, int rope_dims, double rope_base, const int32_t *positions,
                               void *stream) {
    if (!(dtype == LA_DTYPE_BF16 || dtype == LA_DTYPE_F32)) return LA_EUNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return LA_EUNSUPPORTED;
    if (rope_dims <= 0) return LA_EUNSUPPORTED;
    const int rs = check_rope(rope_dims, rope_base, head_dim);
    if (rs != LA_OK) return rs;
    if (batch < 1 || heads < 1) return LA_EINVAL;
    if (!la::decode_grid_ok(batch, heads)) return LA_EUNSUPPORTED;
    if (!q || !k || !v || !o || !positions) return LA_EINVAL;
    if (!la::aligned16(state) || !la::aligned4(positions) || !la::aligned4(slots)) return LA_EINVAL;
    if (slots) {
        if (nslots < 0) return LA_EINVAL;
        if ((int64_t)nslots * heads > (int64_t)INT32_MAX) return LA_EUNSUPPORTED;
        if (nslots > 0 && !state) return LA_EINVAL;
    } else {
        if (!state) return LA_EINVAL;
        nslots = 0;
    }
    return la::launch_decode(q, k, v, state, o, batch, heads, head_dim, dtype, stream, slots, nslots,
                             rope_dims, rope_base, positions) == 0 ? LA_OK : LA_EHIP;
}

const char *lightning_attn_strerror(int status) {
    switch (status) {
        case LA_OK: return "success";
        case LA_EINVAL: return "invalid argument (null pointer with work to do, bad size or alignment)";
        case LA_EUNSUPPORTED: return "unsupported head_dim, block_size, dtype or size";
        case LA_EWORKSPACE: return "workspace missing or smaller than lightning_attn_fwd_workspace_size()";
        case LA_EHIP: return "HIP kernel launch failed";
        case LA_ESCRATCH: return "the call needs more scratch than the allocation-free entry point holds";
        default: return "unknown status";
    }
}

}  // extern "C"
