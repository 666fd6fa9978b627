// la_prefill.hip -- Lightning Attention forward pass on gfx950.
//
// The method (wiki page "MiniMax-01 Lightning Attention", section "Lightning
// Attention 设计"; Tencent Cloud article, section 4.1): cut each sequence into
// blocks of B tokens.  Inside a block use the left product
//     O_b^intra = mask(Q_b K_b^T) V_b          (mask keeps j <= i)
// and across blocks the right product with the compact key-value prefix
//     O_b = O_b^intra + Q_b S_b ,   S_b = sum over earlier blocks of K^T V .
//
// Kernels (all on the caller's stream, no host synchronisation):
//   1. k_prep       chunk, sub-chunk and scan-tile offset tables from
//                   cu_seqlens (1 WG; packed input only: for dense input
//                   every sequence has the same counts and the offsets are
//                   products)
//   2. k_summary    U_c = K_c^T V_c for every sub-chunk c of C_s tokens that
//                   precedes a sequence's last chunk (MFMA)
//   3. k_scan_*     fp32 exclusive prefix over sub-chunk states, segmented at
//                   sequence starts, as a three-phase reduce-then-scan across
//                   tiles of sub-chunks (parallel over tiles and the d*d lanes)
//   4. k_fused      per chunk of C tokens (C a multiple of C_s): start from
//                   the prefix at its first sub-chunk and walk the chunk's
//                   blocks; per block the masked Q K^T and P V products (MFMA,
//                   tiles staged in LDS) plus Q S, one store of O, then
//                   S += K_b^T V_b for the next block.
// Chunks (one workgroup each) are sized to fill the chip; the summaries work
// on sub-chunks of at most 16384 tokens so that they have enough workgroups of
// their own, and skip the sequence's last chunk, whose prefix-sum is never needed.
// The intra-block product and the output combine are one kernel: both
// accumulate into the same registers (O^T = V^T P^T + S^T Q^T), so the
// intra-block partial never goes to memory.
#include <hip/hip_runtime.h>

#include <atomic>

#include "la_common.h"
#include "la_internal.h"

namespace la {

struct KParams {
    const void *q, *k, *v;
    void *o;
    const int32_t *cu;      // packed offsets, or nullptr (dense)
    int32_t *chunk_off;     // [nseq + 1] chunks before each sequence
    // longest-first order of the chunk workgroups (packed input; nullptr for
    // dense): perm[r] = sequence of length rank r, rank_off[r] = chunks of the
    // sequences ranked before r
    int32_t *perm;          // [nseq]
    int32_t *rank_off;      // [nseq + 1]
    // the same order as a direct table (packed input; nullptr for dense):
    // slot_tab[2 r], slot_tab[2 r + 1] = sequence and global chunk of slot r
    int32_t *slot_tab;      // [nchunk_ub][2]
    int32_t *sub_off;       // [nseq + 1] sub-chunks before each sequence
    int32_t *tile_off;      // [nseq + 1] scan tiles before each sequence
    int32_t *err;           // set to 1 by k_prep when cu_seqlens is malformed
    float *states;          // [heads][nsub_ub][D*D]
    float *tilesum;         // [heads][ntile_ub][D*D]
    int64_t seq_len;        // dense: per sequence; packed: total tokens
    int64_t chunk;          // tokens per chunk (a multiple of sub)
    int64_t sub;            // tokens per sub-chunk
    int64_t nchunk_ub, nsub_ub, ntile_ub;
    // dense input: chunks, sub-chunk entries and scan tiles per sequence (the
    // same for every sequence, so the offset tables are products)
    int64_t cps, nsps, tps;
    int nseq, heads, group;
    // state handoff: initial states [nseq][heads][D][D] (or nullptr = zero)
    // and final states of the same layout (or nullptr = not wanted).
    // init_mode 0: no initial state; 1: the scan adds it to the prefixes in
    // `states` of sequences of several chunks, and a sequence of one chunk
    // reads it directly; 2: every sequence is one chunk and reads it directly.
    // With a slot table, s_init and s_final are one pool of nslots entries
    // and sequence s uses entry slots[s] (none when out of range).
    const float *s_init;
    float *s_final;
    int init_mode;
    const int32_t *slots;
    int nslots;
    // rotary position embedding of q and k (bf16 kernels with ROPE set):
    // rope_dims rotated dims, base frequency, and the position of each
    // sequence's first token (pos0[s], or 0 when pos0 is nullptr)
    const int32_t *pos0;
    double rope_base;
    int rope_dims;
};

// ------------------------------------------------------------------ units

struct Unit {
    int64_t base;   // element offset of token 0 of this (sequence, head)
    int64_t len;    // tokens
};

template <int D>
__device__ __forceinline__ Unit unit_of(const KParams &p, int s, int h) {
    Unit u;
    if (p.cu == nullptr) {
        u.base = ((int64_t)s * p.heads + h) * p.seq_len * D;
        u.len = p.seq_len;
    } else {
        int64_t b = p.cu[s], e = p.cu[s + 1];
        u.base = ((int64_t)h * p.seq_len + b) * D;
        u.len = e - b;
    }
    return u;
}

// Largest s in [0, n) with off[s] <= x (off non-decreasing, off[0] = 0).
__device__ __forceinline__ int find_seg(const int32_t *off, int n, int64_t x) {
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if ((int64_t)off[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

// Chunks, sub-chunk entries and scan tiles before sequence s.  Packed input:
// the tables k_prep builds from cu_seqlens; dense input: every sequence has
// the same counts, so no tables are built and these are products.
__device__ __forceinline__ int64_t chunk_off(const KParams &p, int s) {
    return p.cu ? (int64_t)p.chunk_off[s] : (int64_t)s * p.cps;
}
__device__ __forceinline__ int64_t sub_off(const KParams &p, int s) {
    return p.cu ? (int64_t)p.sub_off[s] : (int64_t)s * p.nsps;
}
__device__ __forceinline__ int64_t tile_off(const KParams &p, int s) {
    return p.cu ? (int64_t)p.tile_off[s] : (int64_t)s * p.tps;
}
// The sequence of sub-chunk entry x, resp. scan tile x (x below the total).
__device__ __forceinline__ int seq_of_sub(const KParams &p, int64_t x) {
    return p.cu ? find_seg(p.sub_off, p.nseq, x) : (int)(x / p.nsps);
}
__device__ __forceinline__ int seq_of_tile(const KParams &p, int64_t x) {
    return p.cu ? find_seg(p.tile_off, p.nseq, x) : (int)(x / p.tps);
}

// The (head, chunk, sequence) of a chunk workgroup, or false when the
// workgroup has no chunk.  Workgroups are taken in dispatch order with the
// head varying fastest, so all heads of one chunk slot start together; with
// a ranking (packed input) the slots go to the chunks of the longest
// sequences first, so that a long sequence's chunks do not start last and
// hold a few CUs after the others have finished.
__device__ __forceinline__ bool chunk_of_block(const KParams &p, int &h, int64_t &gch, int &s) {
    const int64_t lin = (int64_t)blockIdx.x + (int64_t)gridDim.x * blockIdx.y;
    h = (int)(lin % p.heads);
    const int64_t slot = lin / p.heads;
    if (slot >= chunk_off(p, p.nseq)) return false;
    if (p.slot_tab != nullptr) {        // one load instead of a search over the ranking
        const int2 e = reinterpret_cast<const int2 *>(p.slot_tab)[slot];
        s = e.x;
        gch = e.y;
    } else {                            // dense: every sequence has the same chunk count
        gch = slot;
        s = (int)(gch / p.cps);
    }
    return true;
}

// State entry of sequence s: s itself, or with a slot table slots[s]; -1 when
// the slot is out of range (no state read or written: the sequence starts
// from zero and its final state is dropped).
__device__ __forceinline__ int64_t state_entry(const KParams &p, int s) {
    if (p.slots == nullptr) return s;
    const int sl = p.slots[s];
    return (sl < 0 || sl >= p.nslots) ? -1 : sl;
}

// Source of the state at the start of chunk cl (chunk-local index) of
// sequence s, head h, or nullptr for zero: the scanned prefix in `states` at
// the chunk's first sub-chunk (which includes a carried-in initial state when
// one was given), or for a sequence of one chunk the initial state itself
// (read and then overwritten by the same workgroup, so an initial state that
// is also the final state's memory is safe; with several chunks the scan
// copies it first, since the last chunk's workgroup writes the final state).
template <int D>
__device__ __forceinline__ const float *chunk_start_state(const KParams &p, int s, int h, int64_t cl) {
    if (p.init_mode == 2 || chunk_off(p, s + 1) - chunk_off(p, s) == 1) {
        const int64_t e = p.init_mode == 0 ? -1 : state_entry(p, s);
        return e < 0 ? nullptr : p.s_init + (e * p.heads + h) * (D * D);
    }
    if (p.init_mode == 0 && cl == 0) return nullptr;
    const int64_t gsub = sub_off(p, s) + cl * (p.chunk / p.sub);
    return p.states + ((int64_t)h * p.nsub_ub + gsub) * (D * D);
}

// Sub-chunk gsub of sequence s, or -1 when its summary is not needed (it lies
// in the sequence's last chunk): its first token otherwise.
__device__ __forceinline__ int64_t sub_first_token(const KParams &p, int s, int64_t gsub) {
    const int64_t t0 = (gsub - sub_off(p, s)) * p.sub;
    const int64_t nc = chunk_off(p, s + 1) - chunk_off(p, s);
    return t0 >= (nc - 1) * p.chunk ? -1 : t0;
}

// Final state of (s, h) when the caller asked for it and chunk gch is the
// sequence's last: the workgroup of that chunk writes it; else nullptr.
template <int D>
__device__ __forceinline__ float *final_state_dst(const KParams &p, int s, int h, int64_t gch) {
    if (p.s_final == nullptr || gch + 1 != chunk_off(p, s + 1)) return nullptr;
    const int64_t e = state_entry(p, s);
    return e < 0 ? nullptr : p.s_final + (e * p.heads + h) * (D * D);
}

// Final state of sequences with no tokens: the initial state (or zero).
// (Not launched with a slot table: there the entry is updated in place.)
template <int D>
__global__ __launch_bounds__(256) void k_state_empty(KParams p) {
    const int s = blockIdx.x, h = blockIdx.y;
    const int64_t L = p.cu ? (int64_t)p.cu[s + 1] - p.cu[s] : p.seq_len;
    if (L != 0) return;
    float *dst = p.s_final + ((int64_t)s * p.heads + h) * (D * D);
    const float *src = p.s_init ? p.s_init + ((int64_t)s * p.heads + h) * (D * D) : nullptr;
    for (int e = threadIdx.x; e < D * D; e += 256) dst[e] = src ? src[e] : 0.f;
}

// -------------------------------------------------------------- k_prep
// chunk_off[s] = sum_{s' < s} nc_s', nc = ceil(L / C) chunks of a sequence;
// sub_off[s] = sum ns_s', where ns = (nc - 1) C / C_s + 1 sub-chunk entries
// when nc >= 2 (the summaries of every chunk but the last, and one entry for
// the last chunk's start prefix) and 0 for a sequence of one chunk, which
// needs no prefix; tile_off[s] = sum ceil(ns_s' / G).
constexpr int kPrepThreads = 1024;
constexpr int kSortMax = 4096;   // sequences ranked by length for the fused grid

__global__ __launch_bounds__(kPrepThreads) void k_prep(KParams p) {
    __shared__ int64_t sc[kPrepThreads], su[kPrepThreads], st[kPrepThreads];
    const int t = threadIdx.x;
    const int per = (p.nseq + kPrepThreads - 1) / kPrepThreads;
    const int s0 = t * per, s1 = min(p.nseq, s0 + per);
    // cu_seqlens must start at 0, never decrease and end at the token count.
    // A malformed table must not send any kernel out of bounds: every
    // sequence is then given no chunks (nothing is computed) and the error
    // flag is raised.
    if (p.cu != nullptr) {
        int bad = 0;
        for (int s = s0; s < s1; ++s) bad |= p.cu[s + 1] < p.cu[s];
        if (t == 0) bad |= p.cu[0] != 0 || (int64_t)p.cu[p.nseq] != p.seq_len;
        if (__syncthreads_or(bad)) {
            for (int s = s0; s < s1; ++s) {
                p.chunk_off[s] = 0; p.sub_off[s] = 0; p.tile_off[s] = 0;
                if (p.perm) { p.perm[s] = s; p.rank_off[s] = 0; }
            }
            if (t == 0) {
                p.chunk_off[p.nseq] = 0; p.sub_off[p.nseq] = 0; p.tile_off[p.nseq] = 0;
                if (p.rank_off) p.rank_off[p.nseq] = 0;
                if (p.err) p.err[0] = 1;
            }
            return;
        }
        if (t == 0 && p.err) p.err[0] = 0;
    }
    auto counts = [&](int s, int64_t &nc, int64_t &ns, int64_t &ng) {
        const int64_t L = p.cu ? (int64_t)p.cu[s + 1] - p.cu[s] : p.seq_len;
        nc = (L + p.chunk - 1) / p.chunk;
        ns = nc >= 2 ? (nc - 1) * (p.chunk / p.sub) + 1 : 0;
        ng = (ns + p.group - 1) / p.group;
    };
    int64_t c = 0, u = 0, g = 0;
    for (int s = s0; s < s1; ++s) {
        int64_t nc, ns, ng;
        counts(s, nc, ns, ng);
        c += nc; u += ns; g += ng;
    }
    sc[t] = c; su[t] = u; st[t] = g;
    __syncthreads();
    for (int d = 1; d < kPrepThreads; d <<= 1) {   // inclusive Hillis-Steele scan
        const int64_t a = t >= d ? sc[t - d] : 0, b = t >= d ? su[t - d] : 0, e = t >= d ? st[t - d] : 0;
        __syncthreads();
        sc[t] += a; su[t] += b; st[t] += e;
        __syncthreads();
    }
    c = t ? sc[t - 1] : 0;
    u = t ? su[t - 1] : 0;
    g = t ? st[t - 1] : 0;
    for (int s = s0; s < s1; ++s) {
        p.chunk_off[s] = (int32_t)c;
        p.sub_off[s] = (int32_t)u;
        p.tile_off[s] = (int32_t)g;
        int64_t nc, ns, ng;
        counts(s, nc, ns, ng);
        c += nc; u += ns; g += ng;
    }
    if (t == kPrepThreads - 1) {
        p.chunk_off[p.nseq] = (int32_t)sc[t];
        p.sub_off[p.nseq] = (int32_t)su[t];
        p.tile_off[p.nseq] = (int32_t)st[t];
    }
    if (p.perm == nullptr) return;

    // Longest-first ranking of the sequences (bitonic sort of (length, index)
    // keys in LDS, up to kSortMax sequences; beyond that the natural order),
    // then rank_off = exclusive prefix of the chunk counts in rank order.
    __shared__ uint64_t key[kSortMax];
    const int n = p.nseq;
    const bool sorted = n <= kSortMax;
    if (sorted) {
        int np2 = 1;
        while (np2 < n) np2 <<= 1;
        for (int i = t; i < np2; i += kPrepThreads) {
            const int64_t L = i < n ? (int64_t)p.cu[i + 1] - p.cu[i] : 0;
            key[i] = i < n ? ((uint64_t)(INT32_MAX - L) << 32) | (uint32_t)i : ~0ull;
        }
        __syncthreads();
        for (int k = 2; k <= np2; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = t; i < np2; i += kPrepThreads) {
                    const int ixj = i ^ j;
                    if (ixj > i) {
                        const uint64_t a = key[i], b = key[ixj];
                        if ((a > b) == ((i & k) == 0)) { key[i] = b; key[ixj] = a; }
                    }
                }
                __syncthreads();
            }
        }
    }
    auto seq_at = [&](int r) { return sorted ? (int)(uint32_t)key[r] : r; };
    int64_t cr = 0;
    for (int r = s0; r < s1; ++r) {
        int64_t nc, ns, ng;
        counts(seq_at(r), nc, ns, ng);
        cr += nc;
    }
    __syncthreads();
    sc[t] = cr;
    __syncthreads();
    for (int d = 1; d < kPrepThreads; d <<= 1) {
        const int64_t a = t >= d ? sc[t - d] : 0;
        __syncthreads();
        sc[t] += a;
        __syncthreads();
    }
    cr = t ? sc[t - 1] : 0;
    for (int r = s0; r < s1; ++r) {
        const int sq = seq_at(r);
        p.perm[r] = sq;
        p.rank_off[r] = (int32_t)cr;
        int64_t nc, ns, ng;
        counts(sq, nc, ns, ng);
        // chunk_off was written by other threads before the barriers above
        const int32_t c0 = p.chunk_off[sq];
        for (int64_t i = 0; i < nc; ++i) {
            p.slot_tab[2 * (cr + i)] = sq;
            p.slot_tab[2 * (cr + i) + 1] = c0 + (int32_t)i;
        }
        cr += nc;
    }
    if (t == kPrepThreads - 1) p.rank_off[n] = (int32_t)sc[t];
}

// ---------------------------------------------------------- tile config

template <typename T, int D, int BLK, int NWAVES = 8>
struct Cfg {
    static constexpr int ES = Elem<T>::kBytes;
    static constexpr int NW = NWAVES, NT = NW * kWave;
    static constexpr int TJ = ES == 2 ? 64 : 32;        // K/V tokens per LDS tile
    static constexpr int EPC = 16 / ES;                 // elements per 16-byte chunk
    static constexpr int KR_ROW = D * ES;               // row-major K row bytes
    static constexpr int KT_ROW = TJ * ES;              // transposed row bytes (128)
    static constexpr int ST_ROW = D * ES;
    static constexpr int KR_BYTES = TJ * KR_ROW;
    static constexpr int KT_BYTES = D * KT_ROW;
    static constexpr int ST_BYTES = D * ST_ROW;
    static constexpr int NP = (TJ / 4) * (D / EPC);     // 4-token patches per tensor tile
    static constexpr int DT = D / 16;                   // 16-wide tiles along d
    static constexpr int KC = D / 32;                   // 32-wide k steps along d
    // state tiles per wave: SA x SB of the DT x DT grid
    static constexpr int SA = NW == 16 ? (D == 128 ? 2 : 1) : (D == 128 ? 2 : 1);
    static constexpr int SB = NW == 16 ? (D == 128 ? 2 : 1) : (D == 128 ? 4 : 2);
    static constexpr int AW = DT / SA;                  // waves along a
    // row slabs (16 rows) of a block handled per wave, and the column split
    static constexpr int NSLAB = BLK / 16;
    static constexpr int NSW = NW == 16 ? 1 : (BLK == 64 ? 1 : 2);
    static constexpr int CSPLIT = NW * NSW / NSLAB;     // waves sharing one slab (by columns)
    static constexpr int NCT = DT / CSPLIT;             // 16-wide output column tiles per wave
    static_assert(NP <= 256, "patch mapping");
    static_assert(AW * (DT / SB) == NW, "state split");
    static_assert(BLK % TJ == 0, "tile");
    static_assert(CSPLIT >= 1 && DT % CSPLIT == 0, "column split");
};

// Row slab (0..BLK/16-1) handled as slab `s` by wave w.  Eight waves: pairs of
// slabs from both ends of the block so that every wave does the same causal
// work.  Sixteen waves: one slab each; the four waves of a SIMD (w, w+4, ...)
// then hold one slab from each quarter of the block.
template <int BLK, int NW = 8>
__device__ __forceinline__ int slab_of(int w, int s) {
    if constexpr (NW == 16) return w % (BLK / 16);
    else if constexpr (BLK == 256) return s == 0 ? w : 15 - w;
    else if constexpr (BLK == 128) return s == 0 ? (w & 3) : 7 - (w & 3);
    else return w & 3;
}

// First 16-wide output column tile of wave w.
template <int BLK, int NW, int NCT>
__device__ __forceinline__ int col_tile0(int w) {
    constexpr int NSLAB = BLK / 16;
    if constexpr (NW == 16) return (w / NSLAB) * NCT;
    else return BLK == 256 ? 0 : (w >> 2) * NCT;
}

// ------------------------------------------------------ tile staging
// Each of the first NP threads owns a 4-token x 16-byte patch of K, the
// threads [256, 256 + NP) the same patch of V.  The patch is loaded with four
// 16-byte global loads (coalesced along d), written to LDS row-major (K
// only, for Q K^T) and transposed (token-contiguous rows, for the products
// that reduce over tokens).
template <typename T, int D>
struct Patch {
    u32x4_t x[4];
};

template <typename T, int D, int BLK>
__device__ __forceinline__ void patch_load(Patch<T, D> &pt, const T *kbase, const T *vbase,
                                           int64_t tok0, int64_t tend) {
    using C = Cfg<T, D, BLK>;
    const int t = threadIdx.x;
    const bool isk = t < C::NP;
    const bool isv = t >= 256 && t < 256 + C::NP;
    const int pi = isk ? t : t - 256;
    const int tg = pi / (D / C::EPC), ch = pi % (D / C::EPC);
    const T *src = isk ? kbase : vbase;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t tok = tok0 + 4 * tg + r;
        const bool ok = (isk || isv) && tok < tend;
        pt.x[r] = ok ? *reinterpret_cast<const u32x4_t *>(src + tok * D + ch * C::EPC)
                     : u32x4_t{0u, 0u, 0u, 0u};
    }
}

template <typename T, int D, int BLK, bool kWithRowMajor>
__device__ __forceinline__ void patch_store(const Patch<T, D> &pt, char *kr, char *kt, char *vt) {
    using C = Cfg<T, D, BLK>;
    const int t = threadIdx.x;
    const bool isk = t < C::NP;
    const bool isv = t >= 256 && t < 256 + C::NP;
    if (!isk && !isv) return;
    const int pi = isk ? t : t - 256;
    const int tg = pi / (D / C::EPC), ch = pi % (D / C::EPC);
    if (kWithRowMajor && isk) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<u32x4_t *>(kr + LdsRows<C::KR_ROW>::off(4 * tg + r, ch * 16)) = pt.x[r];
    }
    char *dst = isk ? kt : vt;
    if constexpr (C::ES == 2) {
        // element e of token r sits in dword e/2, half e%2, of pt.x[r]
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int dw = e >> 1;
            uint32_t lo, hi;
            if (e & 1) {
                lo = (pt.x[0][dw] >> 16) | (pt.x[1][dw] & 0xffff0000u);
                hi = (pt.x[2][dw] >> 16) | (pt.x[3][dw] & 0xffff0000u);
            } else {
                lo = (pt.x[0][dw] & 0xffffu) | (pt.x[1][dw] << 16);
                hi = (pt.x[2][dw] & 0xffffu) | (pt.x[3][dw] << 16);
            }
            *reinterpret_cast<u32x2_t *>(dst + LdsRows<C::KT_ROW>::off(ch * 8 + e, 4 * tg * 2)) =
                u32x2_t{lo, hi};
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            *reinterpret_cast<u32x4_t *>(dst + LdsRows<C::KT_ROW>::off(ch * 4 + e, 4 * tg * 4)) =
                u32x4_t{pt.x[0][e], pt.x[1][e], pt.x[2][e], pt.x[3][e]};
    }
}

// Rotary embedding for the fp32 kernels.  Frequency in turns of pair i.
__device__ __forceinline__ double rope_f_pair(const KParams &p, int i) {
    return (0.5 / 3.14159265358979323846) * exp2(-2.0 * i / p.rope_dims * log2(p.rope_base));
}

// Rotate the K rows of a patch (the first NP threads hold 4 tokens x one
// 16-byte chunk ch, dims 4 ch .. 4 ch + 3, of K; the partner chunk ch ^ HC,
// HC = D / 16, sits in lane l ^ HC of the same wave).  pos0: position of
// token 0 of the unit; tok0: the patch tile's first token.
template <typename T, int D, int BLK>
__device__ __forceinline__ void rope_patch(Patch<T, D> &pt, const KParams &p, int64_t pos0, int64_t tok0) {
    using C = Cfg<T, D, BLK>;
    static_assert(sizeof(T) == 4, "fp32 patches");
    static_assert(C::NP % 64 == 0, "whole waves of K patch threads");
    constexpr int HC = D / 16;
    const int t = threadIdx.x;
    if (t >= C::NP) return;                         // wave-uniform
    const int tg = t / (D / C::EPC), ch = t % (D / C::EPC);
    const bool rot = ch < 2 * HC, first = ch < HC;
    const double f0 = rope_f_pair(p, 4 * (ch % HC)), rho = rope_rho(p.rope_base, p.rope_dims);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const double pos = (double)(pos0 + tok0 + 4 * tg + r);
        double f = f0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = __uint_as_float(pt.x[r][e]);
            const float y = __uint_as_float((uint32_t)__shfl_xor((int)pt.x[r][e], HC));
            float cs, sn;
            rope_cs(pos, f, cs, sn);
            f *= rho;
            if (rot) pt.x[r][e] = __float_as_uint(first ? x * cs - y * sn : y * sn + x * cs);
        }
    }
}

// S[ia][ib] += K^T V over one LDS tile (TJ tokens).  Wave w owns the state
// tiles a in [a0, a0+SA), b in [b0, b0+SB) (16 x 16 each).
template <typename T, int D, int BLK, int SA, int SB>
__device__ __forceinline__ void state_update(f32x4_t (&S)[SA][SB], const char *kt, const char *vt,
                                             int a0, int b0) {
    using C = Cfg<T, D, BLK>;
    static_assert(SA == C::SA && SB == C::SB, "state split");
    const int l = lane_id(), c = l & 15, g = l >> 4;
#pragma unroll
    for (int jg = 0; jg < C::TJ / 32; ++jg) {
        Frag<T> A[C::SA], B[C::SB];
#pragma unroll
        for (int ia = 0; ia < C::SA; ++ia)
            A[ia] = lds_read8<T, C::KT_ROW>(kt, (a0 + ia) * 16 + c, jg * 32 + 8 * g);
#pragma unroll
        for (int ib = 0; ib < C::SB; ++ib)
            B[ib] = lds_read8<T, C::KT_ROW>(vt, (b0 + ib) * 16 + c, jg * 32 + 8 * g);
#pragma unroll
        for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
            for (int ib = 0; ib < C::SB; ++ib) mma(S[ia][ib], A[ia], B[ib]);
    }
}

// --------------------------------------------------------- k_summary
// states[h][sub-chunk] = K_c^T V_c  (fp32, row a = key dim, column b = value dim)
template <typename T, int D, int BLK, bool ROPE>
__global__ __launch_bounds__(512, 2) void k_summary(KParams p) {
    using C = Cfg<T, D, BLK>;
    __shared__ __attribute__((aligned(16))) char lds[2][2 * C::KT_BYTES];
    const int h = blockIdx.y;
    const int64_t gch = blockIdx.x;
    if (gch >= sub_off(p, p.nseq)) return;
    const int s = seq_of_sub(p, gch);
    const int64_t t0 = sub_first_token(p, s, gch);
    if (t0 < 0) return;                              // in the sequence's last chunk: not needed
    const Unit u = unit_of<D>(p, s, h);
    const int64_t t1 = min(u.len, t0 + p.sub);
    const T *kb = reinterpret_cast<const T *>(p.k) + u.base;
    const T *vb = reinterpret_cast<const T *>(p.v) + u.base;

    const int w = wave_id(), l = lane_id(), c = l & 15, g = l >> 4;
    const int a0 = C::SA * (w % C::AW), b0 = C::SB * (w / C::AW);
    f32x4_t S[C::SA][C::SB];
#pragma unroll
    for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
        for (int ib = 0; ib < C::SB; ++ib) S[ia][ib] = zero4();

    const int64_t ntile = (t1 - t0 + C::TJ - 1) / C::TJ;
    const int64_t pos0 = ROPE && p.pos0 ? p.pos0[s] : 0;
    Patch<T, D> pt;
    patch_load<T, D, BLK>(pt, kb, vb, t0, t1);
    if constexpr (ROPE) rope_patch<T, D, BLK>(pt, p, pos0, t0);
    patch_store<T, D, BLK, false>(pt, nullptr, lds[0], lds[0] + C::KT_BYTES);
    __syncthreads();
    for (int64_t it = 0; it < ntile; ++it) {
        const int buf = it & 1;
        if (it + 1 < ntile) {
            patch_load<T, D, BLK>(pt, kb, vb, t0 + (it + 1) * C::TJ, t1);
            if constexpr (ROPE) rope_patch<T, D, BLK>(pt, p, pos0, t0 + (it + 1) * C::TJ);
        }
        state_update<T, D, BLK, C::SA, C::SB>(S, lds[buf], lds[buf] + C::KT_BYTES, a0, b0);
        if (it + 1 < ntile)
            patch_store<T, D, BLK, false>(pt, nullptr, lds[buf ^ 1], lds[buf ^ 1] + C::KT_BYTES);
        __syncthreads();
    }
    float *dst = p.states + ((int64_t)h * p.nsub_ub + gch) * (D * D);
#pragma unroll
    for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
        for (int ib = 0; ib < C::SB; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[((a0 + ia) * 16 + 4 * g + r) * D + (b0 + ib) * 16 + c] = S[ia][ib][r];
}

// ------------------------------------------------------------- scans
// Exclusive prefix over the sub-chunks of every (sequence, head), in place
// on `states`.  Lanes are the d*d state entries; tiles of G sub-chunks are
// reduced (A), the tile totals scanned per sequence (B), and each tile
// rescanned from its prefix (C).  With every sequence inside one tile only
// phase C runs.  Only chunk starts are read back, so C writes the prefix
// there and nowhere else.  (A sequence's last entry, the last chunk's start,
// holds no summary; it only reaches the tile total of the last tile, which
// no prefix uses.)
constexpr int kScanThreads = 256;

template <int D>
__global__ __launch_bounds__(kScanThreads) void k_scan_reduce(KParams p) {
    const int h = blockIdx.z;
    const int64_t tile = blockIdx.x;
    if (tile >= tile_off(p, p.nseq)) return;
    const int s = seq_of_tile(p, tile);
    const int64_t c0 = sub_off(p, s) + (tile - tile_off(p, s)) * p.group;
    const int64_t c1 = min(sub_off(p, s + 1), c0 + p.group);
    const int e = blockIdx.y * kScanThreads + threadIdx.x;
    const float *src = p.states + (int64_t)h * p.nsub_ub * (D * D) + e;
    float acc = 0.f;
    for (int64_t c = c0; c < c1; ++c) acc += src[c * (D * D)];
    p.tilesum[((int64_t)h * p.ntile_ub + tile) * (D * D) + e] = acc;
}

// (B runs on the tile grid: the workgroup of a sequence's first tile scans
// that sequence's tile totals, the others have nothing to do.)
template <int D>
__global__ __launch_bounds__(kScanThreads) void k_scan_tiles(KParams p) {
    const int h = blockIdx.z;
    const int64_t tile = blockIdx.x;
    if (tile >= tile_off(p, p.nseq)) return;
    const int s = seq_of_tile(p, tile);
    if (tile != tile_off(p, s)) return;
    const int e = blockIdx.y * kScanThreads + threadIdx.x;
    float *ts = p.tilesum + (int64_t)h * p.ntile_ub * (D * D) + e;
    float run = 0.f;
    for (int64_t t = tile_off(p, s); t < tile_off(p, s + 1); ++t) {
        const float x = ts[t * (D * D)];
        ts[t * (D * D)] = run;
        run += x;
    }
}

template <int D>
__global__ __launch_bounds__(kScanThreads) void k_scan_apply(KParams p, int use_tiles) {
    const int h = blockIdx.z;
    const int64_t tile = blockIdx.x;
    if (tile >= tile_off(p, p.nseq)) return;
    const int s = seq_of_tile(p, tile);
    const int64_t c0 = sub_off(p, s) + (tile - tile_off(p, s)) * p.group;
    const int64_t c1 = min(sub_off(p, s + 1), c0 + p.group);
    const int e = blockIdx.y * kScanThreads + threadIdx.x;
    float *st = p.states + (int64_t)h * p.nsub_ub * (D * D) + e;
    float run = use_tiles ? p.tilesum[((int64_t)h * p.ntile_ub + tile) * (D * D) + e] : 0.f;
    if (p.s_init) {                                  // carried-in state
        const int64_t se = state_entry(p, s);
        if (se >= 0) run += p.s_init[(se * p.heads + h) * (D * D) + e];
    }
    const int64_t per = p.chunk / p.sub;
    int64_t j = (c0 - sub_off(p, s)) % per;           // sub-chunk index within its chunk
    for (int64_t c = c0; c < c1; ++c) {
        const float x = st[c * (D * D)];
        if (j == 0) st[c * (D * D)] = run;
        run += x;
        if (++j == per) j = 0;
    }
}

// fp32 state tiles of a wave (its SA x SB grid of 16 x 16 tiles at a0, b0;
// lane (c, g) holds rows 4g .. 4g+3, column c of each) to global memory.
template <int D, int SA, int SB>
__device__ __forceinline__ void store_state(float *dst, const f32x4_t (&S)[SA][SB], int a0, int b0, int c, int g) {
#pragma unroll
    for (int ia = 0; ia < SA; ++ia)
#pragma unroll
        for (int ib = 0; ib < SB; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[((a0 + ia) * 16 + 4 * g + r) * D + (b0 + ib) * 16 + c] = S[ia][ib][r];
}

// ----------------------------------------------------------- k_fused
template <typename T, int D, int BLK, bool ROPE>
__global__ __launch_bounds__(512, 1) void k_fused(KParams p) {
    using C = Cfg<T, D, BLK>;
    constexpr int NBUF = (C::ES == 4 && D == 128) ? 1 : 2;
    constexpr int BUF = C::KR_BYTES + 2 * C::KT_BYTES;
    __shared__ __attribute__((aligned(16))) char lds[NBUF * BUF + C::ST_BYTES];
    char *const st = lds + NBUF * BUF;

    int h, s;
    int64_t gch;
    if (!chunk_of_block(p, h, gch, s)) return;
    const Unit u = unit_of<D>(p, s, h);
    const int64_t cl = gch - chunk_off(p, s);
    const int64_t t0 = cl * p.chunk;
    const int64_t t1 = min(u.len, t0 + p.chunk);
    const T *qb = reinterpret_cast<const T *>(p.q) + u.base;
    const T *kb = reinterpret_cast<const T *>(p.k) + u.base;
    const T *vb = reinterpret_cast<const T *>(p.v) + u.base;
    T *ob = reinterpret_cast<T *>(p.o) + u.base;

    const int w = wave_id(), l = lane_id(), c = l & 15, g = l >> 4;
    const int a0 = C::SA * (w % C::AW), b0 = C::SB * (w / C::AW);
    const int ct0 = C::CSPLIT == 1 ? 0 : (w >> 2) * C::NCT;

    // ---- state at the chunk start (exclusive prefix from the scan)
    f32x4_t S[C::SA][C::SB];
    float *const fdst = final_state_dst<D>(p, s, h, gch);
    {
        const float *src = chunk_start_state<D>(p, s, h, cl);
#pragma unroll
        for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
            for (int ib = 0; ib < C::SB; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[ia][ib][r] = src ? src[((a0 + ia) * 16 + 4 * g + r) * D + (b0 + ib) * 16 + c] : 0.f;
#pragma unroll
        for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
            for (int ib = 0; ib < C::SB; ++ib)
                lds_write4<T, C::ST_ROW>(st, (b0 + ib) * 16 + c, (a0 + ia) * 16 + 4 * g, S[ia][ib]);
    }

    const int64_t nblk = (t1 - t0 + BLK - 1) / BLK;
    const int64_t pos0 = ROPE && p.pos0 ? p.pos0[s] : 0;
    Patch<T, D> pt;
    patch_load<T, D, BLK>(pt, kb, vb, t0, t1);
    if constexpr (ROPE) rope_patch<T, D, BLK>(pt, p, pos0, t0);
    patch_store<T, D, BLK, true>(pt, lds, lds + C::KR_BYTES, lds + C::KR_BYTES + C::KT_BYTES);

    // Q fragments of this wave's row slabs: row 16*slab + c, d = 32*kc + 8g .. +7
    // (with ROPE rotated once loaded: for d = 128 dims 8g + m of group 0 pair
    // with group 1's in the same lane; for d = 64 with lane l ^ 32's)
    Frag<T> Q[C::NSW][C::KC];
    auto load_q = [&](int64_t tb) {
#pragma unroll
        for (int si = 0; si < C::NSW; ++si) {
            const int64_t row = tb + 16 * slab_of<BLK>(w, si) + c;
            const bool ok = row < t1;
#pragma unroll
            for (int kc = 0; kc < C::KC; ++kc)
                Q[si][kc] = gload8<T>(qb + row * D + kc * 32 + 8 * g, ok);
            if constexpr (ROPE) {
                static_assert(sizeof(T) == 4, "fp32 fragments");
                const double pos = (double)(pos0 + row), rho = rope_rho(p.rope_base, p.rope_dims);
                double f = rope_f_pair(p, D == 128 ? 8 * g : 8 * (g & 1));
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    float cs, sn;
                    rope_cs(pos, f, cs, sn);
                    f *= rho;
                    if constexpr (D == 128) {
                        const float x = Q[si][0].f[m], y = Q[si][1].f[m];
                        Q[si][0].f[m] = x * cs - y * sn;
                        Q[si][1].f[m] = x * sn + y * cs;
                    } else {
                        const float x = Q[si][0].f[m];
                        const float y = __shfl_xor(x, 32);
                        Q[si][0].f[m] = g < 2 ? x * cs - y * sn : y * sn + x * cs;
                    }
                }
            }
        }
    };
    load_q(t0);
    __syncthreads();

    int buf = 0;
    for (int64_t bi = 0; bi < nblk; ++bi) {
        const int64_t tb = t0 + bi * BLK;
        const int bl = (int)min((int64_t)BLK, t1 - tb);
        const int ntj = (bl + C::TJ - 1) / C::TJ;
        const bool more = bi + 1 < nblk;

        // ---- inter-block right product with the block-start state: O^T = S^T Q^T
        f32x4_t O[C::NSW][C::NCT];
#pragma unroll
        for (int si = 0; si < C::NSW; ++si)
#pragma unroll
            for (int t = 0; t < C::NCT; ++t) O[si][t] = zero4();
#pragma unroll
        for (int t = 0; t < C::NCT; ++t)
#pragma unroll
            for (int kc = 0; kc < C::KC; ++kc) {
                const Frag<T> A = lds_read8<T, C::ST_ROW>(st, (ct0 + t) * 16 + c, kc * 32 + 8 * g);
#pragma unroll
                for (int si = 0; si < C::NSW; ++si) mma(O[si][t], A, Q[si][kc]);
            }

        for (int jt = 0; jt < ntj; ++jt) {
            const char *kr = lds + buf * BUF;
            const char *kt = kr + C::KR_BYTES;
            const char *vt = kt + C::KT_BYTES;
            // prefetch the next tile of the chunk (next block's first tile at the end)
            const bool last = jt + 1 == ntj;
            const bool nxt = !last || more;
            const int64_t ntok = last ? tb + BLK : tb + (jt + 1) * C::TJ;
            if (nxt) {
                patch_load<T, D, BLK>(pt, kb, vb, ntok, t1);
                if constexpr (ROPE) rope_patch<T, D, BLK>(pt, p, pos0, ntok);
            }

            // ---- intra-block left product for this K/V tile
#pragma unroll
            for (int jg = 0; jg < C::TJ / 32; ++jg) {
                const int jb = jt * C::TJ + jg * 32;      // block-local first token of the group
                f32x4_t P[C::NSW][2];
                bool need[C::NSW], need1[C::NSW];
#pragma unroll
                for (int si = 0; si < C::NSW; ++si) {
                    const int i0 = 16 * slab_of<BLK>(w, si);
                    need[si] = jb <= i0 + 15;
                    need1[si] = jb + 16 <= i0 + 15;
                    P[si][0] = zero4();
                    P[si][1] = zero4();
                }
                // P^T = K Q^T : rows j (this group), columns i (the slab)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    bool any = false;
#pragma unroll
                    for (int si = 0; si < C::NSW; ++si) any |= hh ? need1[si] : need[si];
                    if (!any) continue;
#pragma unroll
                    for (int kc = 0; kc < C::KC; ++kc) {
                        const Frag<T> A = lds_read8<T, C::KR_ROW>(kr, jg * 32 + 16 * hh + c, kc * 32 + 8 * g);
#pragma unroll
                        for (int si = 0; si < C::NSW; ++si)
                            if (hh ? need1[si] : need[si]) mma(P[si][hh], A, Q[si][kc]);
                    }
                }
                Frag<T> PF[C::NSW];
#pragma unroll
                for (int si = 0; si < C::NSW; ++si) {
                    const int i0 = 16 * slab_of<BLK>(w, si);
                    const int i = i0 + c;                          // block-local query row
                    if (need[si] && jb + 31 > i0) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (jb + 4 * g + r > i) P[si][0][r] = 0.f;
                            if (jb + 16 + 4 * g + r > i) P[si][1][r] = 0.f;
                        }
                    }
                    PF[si] = frag_from_f32(P[si][0], P[si][1], T{});
                }
                // O^T += V^T P^T : k-slots (4g..4g+3) and (16+4g..16+4g+3) of the group
                bool anyg = false;
#pragma unroll
                for (int si = 0; si < C::NSW; ++si) anyg |= need[si];
                if (anyg) {
#pragma unroll
                    for (int t = 0; t < C::NCT; ++t) {
                        const Frag<T> A = lds_read4x2<T, C::KT_ROW>(vt, (ct0 + t) * 16 + c,
                                                                    jg * 32 + 4 * g, jg * 32 + 16 + 4 * g);
#pragma unroll
                        for (int si = 0; si < C::NSW; ++si)
                            if (need[si]) mma(O[si][t], A, PF[si]);
                    }
                }
            }
            // Q of this block is dead after the last tile's scores: fetch the next block's
            if (last && more) load_q(tb + BLK);
            // ---- state for the next block of this chunk
            if (more || fdst) state_update<T, D, BLK, C::SA, C::SB>(S, kt, vt, a0, b0);

            if (nxt) {
                if (NBUF == 1) __syncthreads();
                char *nk = lds + (NBUF == 2 ? (buf ^ 1) : 0) * BUF;
                patch_store<T, D, BLK, true>(pt, nk, nk + C::KR_BYTES, nk + C::KR_BYTES + C::KT_BYTES);
            }
            __syncthreads();
            if (NBUF == 2) buf ^= 1;
        }

        // ---- store O: lane holds row (16*slab + c), columns 16*t + 4g .. +3
#pragma unroll
        for (int si = 0; si < C::NSW; ++si) {
            const int64_t row = tb + 16 * slab_of<BLK>(w, si) + c;
            if (row < t1) {
#pragma unroll
                for (int t = 0; t < C::NCT; ++t) store4(ob + row * D + (ct0 + t) * 16 + 4 * g, O[si][t]);
            }
        }
        if (more) {
            // every wave read the old state copy before the tile loop's barriers
#pragma unroll
            for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
                for (int ib = 0; ib < C::SB; ++ib)
                    lds_write4<T, C::ST_ROW>(st, (b0 + ib) * 16 + c, (a0 + ia) * 16 + 4 * g, S[ia][ib]);
            __syncthreads();
        }
    }
    if (fdst) store_state<D, C::SA, C::SB>(fdst, S, a0, b0, c, g);
}

// ================================================================ bf16 path
// K and V tiles are buffer-loaded straight into LDS (no VGPR staging) into a
// ring of stages.  Operands that reduce over d (Q K^T, Q S) are read as rows
// with ds_read_b128; operands that reduce over tokens (P V, K^T V) are read as
// columns with ds_read_b64_tr_b16.  The buffer resources end at the chunk end:
// rows past it load as zeros, so they add nothing.
//
// LDS layout of a bf16 matrix with ROWS rows (tokens, or state rows):
// 32-element (64-byte) column blocks, each stored row by row, with the four
// 16-byte chunks of a 64-byte sub-row rotated by XOR with swz(row), which is
// 2 when bit 2 of the row is set and 0 otherwise:
//     byte(row, e) = (e / 32) * ROWS * 64 + row * 64
//                    + (((e % 32) / 8) ^ swz(row)) * 16 + (e % 8) * 2 .
// Every operand read below is then a lane-constant base plus a compile-time
// offset (no per-access address arithmetic).  The LDS has 64 four-byte
// banks; an 8-byte read (ds_read_b64_tr_b16) serves 32 lanes per cycle and a
// 16-byte read (ds_read_b128) 16 lanes per cycle.  Measured on gfx950 with
// the bank-conflict counter, this rotation keeps both access shapes used
// here free of conflicts: 16 rows read at one 16-byte chunk (the row reads)
// and 4-row by 4-column pieces read by transposing loads (the column reads).
// (A rotation by (row >> 2) & 3 leaves both of them two-way conflicted.)
template <int ROWS>
struct SubRows {
    static constexpr int BLOCK = ROWS * 64;
    __device__ __forceinline__ static uint32_t swz(uint32_t row) { return (row >> 1) & 2; }
    __device__ __forceinline__ static uint32_t off(uint32_t row, uint32_t e) {
        return (e >> 5) * BLOCK + row * 64 + ((((e & 31) >> 3) ^ swz(row)) << 4) + (e & 7) * 2;
    }
    // Lane base for 8-element row reads (ds_read_b128): row c, elements 8g..8g+7
    // of column block 0; add block * BLOCK + row0 * 64 (row0 a multiple of 16).
    __device__ __forceinline__ static uint32_t row8_base(int c, int g) {
        return c * 64 + ((g ^ swz(c)) << 4);
    }
    // Lane base for column reads (lds_cols8): lane 16g + 4r + q addresses row
    // 4g + r, elements 16 * par + 4q .. +3 of column block 0 (par = parity of
    // the 16-column tile); add block * BLOCK + row0 * 64 (row0 a multiple of 16).
    __device__ __forceinline__ static uint32_t col_base(int l, int par) {
        const int g = l >> 4, r = (l >> 2) & 3, q = l & 3;
        return (4 * g + r) * 64 + (((2 * par + (q >> 1)) ^ swz(4 * g + r)) << 4) + (q & 1) * 8;
    }
};

template <typename P>
__device__ __forceinline__ Frag<bf16_t> ld_row8(const char *p) {
    Frag<bf16_t> f;
    f.u = *reinterpret_cast<const u32x4_t *>(p);
    return f;
}
// Column read: slots 0..3 from rows +0..3 of the lane's group, slots 4..7
// from the rows 16 further down (the k-slot order the score tile uses).
__device__ __forceinline__ Frag<bf16_t> ld_cols8(const char *p) {
    const u32x2_t a0 = lds_read_tr16(p);
    const u32x2_t a1 = lds_read_tr16(p + 16 * 64);
    Frag<bf16_t> f;
    f.u = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
    return f;
}

// S[ia][ib] += K^T V over one tile of TJ tokens.  ka[ia] / vb[ib] are the
// column-read bases of the wave's state rows a and columns b in this stage.
template <int TJ, int SA, int SB>
__device__ __forceinline__ void state_update_tr(f32x4_t (&S)[SA][SB], const char *const (&ka)[SA],
                                                const char *const (&vb)[SB]) {
#pragma unroll
    for (int jg = 0; jg < TJ / 32; ++jg) {
        Frag<bf16_t> A[SA], B[SB];
#pragma unroll
        for (int ia = 0; ia < SA; ++ia) A[ia] = ld_cols8(ka[ia] + jg * 32 * 64);
#pragma unroll
        for (int ib = 0; ib < SB; ++ib) B[ib] = ld_cols8(vb[ib] + jg * 32 * 64);
#pragma unroll
        for (int ia = 0; ia < SA; ++ia)
#pragma unroll
            for (int ib = 0; ib < SB; ++ib) mma(S[ia][ib], A[ia], B[ib]);
    }
}

// Column-read base, inside a tile, of the 16-column tile `ct` (cols 16ct..).
template <int ROWS>
__device__ __forceinline__ uint32_t col_tile_off(int l, int ct) {
    return SubRows<ROWS>::col_base(l, ct & 1) + (ct >> 1) * SubRows<ROWS>::BLOCK;
}

// The K/V ring: one LDS array per stage, so the compiler tracks each
// buffer-to-LDS load by its destination stage.
template <int NST, int SBY>
struct Ring;
template <int SBY>
struct Ring<4, SBY> {
    __device__ __forceinline__ static void get(char *(&s)[4]) {
        __shared__ __attribute__((aligned(16))) char s0[SBY];
        __shared__ __attribute__((aligned(16))) char s1[SBY];
        __shared__ __attribute__((aligned(16))) char s2[SBY];
        __shared__ __attribute__((aligned(16))) char s3[SBY];
        s[0] = s0; s[1] = s1; s[2] = s2; s[3] = s3;
    }
};

template <int SBY>
struct Ring<2, SBY> {
    __device__ __forceinline__ static void get(char *(&s)[2]) {
        __shared__ __attribute__((aligned(16))) char s0[SBY];
        __shared__ __attribute__((aligned(16))) char s1[SBY];
        s[0] = s0; s[1] = s1;
    }
};


// ------------------------------------------------------ k_fused_ring (fp32)
// fp32 with d = 64 (no rotary prologue): k_fused's products over K/V tiles
// that stream through a 4-stage ring of row-major LDS tiles, filled by
// buffer-to-LDS loads three tiles ahead (48 KiB in flight instead of the one
// register-staged tile of k_fused).  Rows are stored with LdsRows' swizzle
// (each lane's global source offset is permuted accordingly), so a stage's
// K tile is itself the row-major operand of the scores.  The products that
// reduce over tokens read transposed tiles: at the top of tile t the patch
// threads transpose tile t + 1 into the second half of its own stage, which
// the barrier at the end of tile t publishes; one barrier per tile.  Every
// tile, loaded or transposed, lives in its compile-time ring stage, so the
// compiler keeps its buffer-to-LDS loads apart and waits only for what a read
// needs.  All global accesses of K and V go through buffer resources that
// end at the chunk end, so tiles past it load as zeros.
template <int BLK>
__global__ __launch_bounds__(512, 1) void k_fused_ring(KParams p) {
    using T = float;
    constexpr int D = 64;
    using C = Cfg<T, D, BLK>;
    constexpr int TJ = C::TJ;                        // 32 tokens per tile
    constexpr int TPB = BLK / TJ;                    // tiles per block (2, 4, 8)
    constexpr int NST = 4, LA = 3;                   // ring stages; tiles requested ahead
    constexpr int RB = D * 4;                        // bytes per token row
    constexpr int TB = TJ * RB;                      // bytes of one tensor tile
    constexpr int SBY = 2 * TB + 2 * C::KT_BYTES;    // stage: K, V tiles, then their transposes
    constexpr int NI = TB / 1024;                    // 1 KiB loads per tensor tile
    constexpr int IPW = 2 * NI / C::NW;              // loads per wave per tile
    static_assert(C::NW == 8 && IPW == 2 && C::KR_ROW == RB && TPB >= 2, "tile split");
    // Blocks of 64 (one row slab per wave, two waves per slab): the two
    // waves of a slab split each tile's keys instead of the output columns,
    // so neither recomputes the other's scores.  Each then holds a partial O
    // for all four column tiles; at the block's end it hands the partner's
    // two column tiles over through LDS (exchange buffer: 2 KiB per wave).
    constexpr bool KS = C::NSW == 1 && C::CSPLIT == 2;
    constexpr int NCO = KS ? 2 * C::NCT : C::NCT;   // O column tiles held per wave
    __shared__ __attribute__((aligned(16))) char st[C::ST_BYTES];
    __shared__ __attribute__((aligned(16))) char xbuf[KS ? C::NW * 2048 : 16];
    char *stages[NST];
    Ring<NST, SBY>::get(stages);

    int h, s;
    int64_t gch;
    if (!chunk_of_block(p, h, gch, s)) return;
    const Unit u = unit_of<D>(p, s, h);
    const int64_t cl = gch - chunk_off(p, s);
    const int64_t t0 = cl * p.chunk;
    const int n = (int)min(u.len - t0, p.chunk);     // tokens of this chunk
    const int64_t t1 = t0 + n;
    const int64_t cb = (u.base + t0 * D) * 4;        // byte offset of its first row
    const uint32_t nbytes = (uint32_t)n * RB;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const char *>(p.k) + cb, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const char *>(p.v) + cb, nbytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<char *>(p.o) + cb, nbytes);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const char *>(p.q) + cb, nbytes);

    const int w = wave_id(), l = lane_id(), c = l & 15, g = l >> 4;
    const int a0 = C::SA * (w % C::AW), b0 = C::SB * (w / C::AW);
    const int ct0 = C::CSPLIT == 1 ? 0 : (w >> 2) * C::NCT;
    const int hk = w >> 2;                           // key half of a tile (key split)
    const int nblk = (n + BLK - 1) / BLK;
    const int ntile = (n + TJ - 1) / TJ;             // tiles holding tokens
    const int nsb = (ntile + NST - 1) / NST;

    // loads: wave instruction gi = w * IPW + ii fills rows 4x .. 4x + 3 of the
    // K (gi < NI) or V tile, x = gi mod NI; lane l brings row 4x + l / 16,
    // the 16-byte chunk that lands at physical chunk l % 16 of the row
    uint32_t dvo[IPW], dlo[IPW];
    __amdgpu_buffer_rsrc_t drs[IPW];
#pragma unroll
    for (int ii = 0; ii < IPW; ++ii) {
        const int gi = w * IPW + ii;
        const bool isv = gi >= NI;
        const int row = 4 * (isv ? gi - NI : gi) + (l >> 4);
        dvo[ii] = (uint32_t)(row * RB + (((l & 15) ^ LdsRows<RB>::swz(row)) << 4));
        dlo[ii] = (isv ? TB : 0) + 1024 * (isv ? gi - NI : gi);
        drs[ii] = isv ? rv : rk;
    }
    auto issue = [&](int tile, char *stage) {
#pragma unroll
        for (int ii = 0; ii < IPW; ++ii) dma_lds16(drs[ii], stage + dlo[ii], dvo[ii], (uint32_t)(tile * TB));
    };
    // transposed copy of a stage's tiles: the patch threads read their
    // 4-token x 16-byte patch of K or V from the stage and write it transposed
    // into the stage's second half
    auto transpose = [&](char *stage) {
        char *tbuf = stage + 2 * TB;
        const int t = threadIdx.x;
        const bool isk = t < C::NP, isv = t >= 256 && t < 256 + C::NP;
        if (!isk && !isv) return;
        const int pi = isk ? t : t - 256;
        const int tg = pi / (D / C::EPC), ch = pi % (D / C::EPC);
        const char *src = stage + (isk ? 0 : TB);
        Patch<T, D> pt;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            pt.x[r] = *reinterpret_cast<const u32x4_t *>(src + LdsRows<RB>::off(4 * tg + r, ch * 16));
        patch_store<T, D, BLK, false>(pt, nullptr, tbuf, tbuf + C::KT_BYTES);
    };

    // ---- state at the chunk start
    f32x4_t S[C::SA][C::SB];
    float *const fdst = final_state_dst<D>(p, s, h, gch);
    {
        const float *src = chunk_start_state<D>(p, s, h, cl);
#pragma unroll
        for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
            for (int ib = 0; ib < C::SB; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[ia][ib][r] = src ? src[((a0 + ia) * 16 + 4 * g + r) * D + (b0 + ib) * 16 + c] : 0.f;
#pragma unroll
        for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
            for (int ib = 0; ib < C::SB; ++ib)
                lds_write4<T, C::ST_ROW>(st, (b0 + ib) * 16 + c, (a0 + ia) * 16 + 4 * g, S[ia][ib]);
    }
    // Q fragments of this wave's row slabs: row 16*slab + c, d = 32*kc + 8g .. +7,
    // by buffer loads that are always issued (rows past the chunk end read as
    // zeros), so the explicit waits below can count them
    Frag<T> Q[C::NSW][C::KC];
    constexpr int QL = 2 * C::NSW * C::KC;           // Q loads per wave per block
    auto load_q = [&](int brow) {                    // the block's first row in the chunk
#pragma unroll
        for (int si = 0; si < C::NSW; ++si) {
            const uint32_t voff = (uint32_t)((brow + 16 * slab_of<BLK>(w, si) + c) * RB + 8 * g * 4);
#pragma unroll
            for (int kc = 0; kc < C::KC; ++kc) {
                const f32x4_t x0 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)voff + kc * 128, 0, 0));
                const f32x4_t x1 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)voff + kc * 128 + 16, 0, 0));
#pragma unroll
                for (int m = 0; m < 4; ++m) { Q[si][kc].f[m] = x0[m]; Q[si][kc].f[4 + m] = x1[m]; }
            }
        }
    };
    load_q(0);
    issue(0, stages[0]);
    issue(1, stages[1]);
    issue(2, stages[2]);
    wait_vm_lgkm0<IPW>();                            // the first two tiles (and Q) have landed
    wg_barrier();
    transpose(stages[0]);
    wait_vm_lgkm0<IPW>();
    wg_barrier();

    // O[si][m]: column tile ct0 + m (with the key split, m = 2, 3 are the
    // partner's column tiles ct0 + 2, ct0 + 3 modulo 4)
    f32x4_t O[C::NSW][NCO];
    using std::integral_constant;
    auto tile = [&](auto J_c, int sb) {
        constexpr int J = decltype(J_c)::value;     // ring stage of the tile
        const int t = sb * NST + J;
        const int bi = t / TPB, jt = t % TPB;
        const int64_t tb = t0 + (int64_t)bi * BLK;   // the block's first token
        const bool more = bi + 1 < nblk;
        const bool block_end = jt == TPB - 1 || t + 1 >= ntile;
        issue(t + LA, stages[(J + LA) % NST]);
        // the next tile has landed (waited for before the barrier that ended
        // the previous tile): its transposed copy, published by this tile's
        // barrier
        transpose(stages[(J + 1) % NST]);
        const char *kr = stages[J];
        const char *kt = stages[J] + 2 * TB;
        const char *vt = kt + C::KT_BYTES;

        if (jt == 0) {
            // ---- inter-block right product with the block-start state: O^T = S^T Q^T
#pragma unroll
            for (int si = 0; si < C::NSW; ++si)
#pragma unroll
                for (int ct = 0; ct < NCO; ++ct) O[si][ct] = zero4();
#pragma unroll
            for (int ct = 0; ct < C::NCT; ++ct)
#pragma unroll
                for (int kc = 0; kc < C::KC; ++kc) {
                    const Frag<T> A = lds_read8<T, C::ST_ROW>(st, (ct0 + ct) * 16 + c, kc * 32 + 8 * g);
#pragma unroll
                    for (int si = 0; si < C::NSW; ++si) mma(O[si][ct], A, Q[si][kc]);
                }
        }
        // ---- intra-block left product for this K/V tile (keys jt*TJ .. of the block)
        const int left = (int)(t1 - tb);             // tokens of the chunk from this block on
        if constexpr (KS) {
            // this wave's 16 keys jh .. jh + 15 of the tile against its slab's
            // rows, then P V over all four column tiles
            const int i0 = 16 * slab_of<BLK>(w, 0);
            const int kmax = i0 < left ? min(i0 + 15, left - 1) : -1;   // last key the slab sees
            const int jh = jt * TJ + 16 * hk;
            if (jh <= kmax) {
                f32x4_t P = zero4();
#pragma unroll
                for (int kc = 0; kc < C::KC; ++kc)
                    mma(P, lds_read8<T, C::KR_ROW>(kr, 16 * hk + c, kc * 32 + 8 * g), Q[0][kc]);
                const int i = i0 + c;                  // block-local query row
                if (jh + 15 > i0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (jh + 4 * g + r > i) P[r] = 0.f;
                }
#pragma unroll
                for (int m = 0; m < NCO; ++m) {
                    // keys 16 hk + 4g .. +3 of the transposed V rows of column tile ct0 + m
                    const f32x4_t a = *reinterpret_cast<const f32x4_t *>(
                        vt + LdsRows<C::KT_ROW>::off(((ct0 + m) & 3) * 16 + c, (16 * hk + 4 * g) * 4));
#pragma unroll
                    for (int r = 0; r < 4; ++r) O[0][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], P[r], O[0][m], 0, 0, 0);
                }
            }
        } else {
            const int jb = jt * TJ;
            f32x4_t P[C::NSW][2];
            bool need[C::NSW], need1[C::NSW];
#pragma unroll
            for (int si = 0; si < C::NSW; ++si) {
                const int i0 = 16 * slab_of<BLK>(w, si);
                const int kmax = i0 < left ? min(i0 + 15, left - 1) : -1;   // last key the slab sees
                need[si] = jb <= kmax;
                need1[si] = jb + 16 <= kmax;
                P[si][0] = zero4();
                P[si][1] = zero4();
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                bool any = false;
#pragma unroll
                for (int si = 0; si < C::NSW; ++si) any |= hh ? need1[si] : need[si];
                if (!any) continue;
#pragma unroll
                for (int kc = 0; kc < C::KC; ++kc) {
                    const Frag<T> A = lds_read8<T, C::KR_ROW>(kr, 16 * hh + c, kc * 32 + 8 * g);
#pragma unroll
                    for (int si = 0; si < C::NSW; ++si)
                        if (hh ? need1[si] : need[si]) mma(P[si][hh], A, Q[si][kc]);
                }
            }
            Frag<T> PF[C::NSW];
#pragma unroll
            for (int si = 0; si < C::NSW; ++si) {
                const int i0 = 16 * slab_of<BLK>(w, si);
                const int i = i0 + c;                  // block-local query row
                if (need[si] && jb + 31 > i0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (jb + 4 * g + r > i) P[si][0][r] = 0.f;
                        if (jb + 16 + 4 * g + r > i) P[si][1][r] = 0.f;
                    }
                }
                PF[si] = frag_from_f32(P[si][0], P[si][1], T{});
            }
            bool anyg = false;
#pragma unroll
            for (int si = 0; si < C::NSW; ++si) anyg |= need[si];
            if (anyg) {
#pragma unroll
                for (int ct = 0; ct < C::NCT; ++ct) {
                    const Frag<T> A = lds_read4x2<T, C::KT_ROW>(vt, (ct0 + ct) * 16 + c, 4 * g, 16 + 4 * g);
#pragma unroll
                    for (int si = 0; si < C::NSW; ++si)
                        if (need[si]) mma(O[si][ct], A, PF[si]);
                }
            }
        }
        // this block's Q is dead after its last tile's scores: fetch the next block's
        const bool q_next = block_end && more;
        if (q_next) load_q((bi + 1) * BLK);
        // ---- state for the next block
        if (more || fdst) state_update<T, D, BLK, C::SA, C::SB>(S, kt, vt, a0, b0);
        if (block_end) {
            if constexpr (KS) {
                // hand the partner (wave w ^ 4, the same slab) its two column
                // tiles of this wave's partial O, and take this wave's from it
                char *xw = xbuf + (w ^ 4) * 2048 + l * 16;
                *reinterpret_cast<f32x4_t *>(xw) = O[0][2];
                *reinterpret_cast<f32x4_t *>(xw + 1024) = O[0][3];
                wait_vm_lgkm0<63>();
                wg_barrier();
                const char *xr = xbuf + w * 2048 + l * 16;
                O[0][0] += *reinterpret_cast<const f32x4_t *>(xr);
                O[0][1] += *reinterpret_cast<const f32x4_t *>(xr + 1024);
            }
            // ---- store O: lane holds row (16*slab + c), columns 16*ct + 4g .. +3
            // (buffer stores from inline asm, outside the compiler's count of
            // outstanding loads; rows past the chunk end are dropped)
#pragma unroll
            for (int si = 0; si < C::NSW; ++si) {
                const uint32_t row = (uint32_t)(bi * BLK + 16 * slab_of<BLK>(w, si) + c);
#pragma unroll
                for (int ct = 0; ct < C::NCT; ++ct)
                    store16(ro, row * RB + ((ct0 + ct) * 16 + 4 * g) * 4, __builtin_bit_cast(u32x4_t, O[si][ct]));
            }
            // the block-start state copy for the next block: every wave read the
            // old one in the block's first tile, before a barrier
            if (more) {
#pragma unroll
                for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
                    for (int ib = 0; ib < C::SB; ++ib)
                        lds_write4<T, C::ST_ROW>(st, (b0 + ib) * 16 + c, (a0 + ia) * 16 + 4 * g, S[ia][ib]);
            }
        }
        // the tile after next has landed: younger are the loads of tile t + 3
        // and the next block's Q (the stores, when younger, only make the
        // wait stricter)
        if (q_next) wait_vm_lgkm0<IPW + QL>();
        else wait_vm_lgkm0<IPW>();
        wg_barrier();
    };

    // tiles past the chunk's last token hold only zeros: the walk stops
    // after the last tile with tokens (every block's O is stored there)
    for (int sb = 0; sb < nsb; ++sb) {
        tile(integral_constant<int, 0>{}, sb);
        if (sb * NST + 1 >= ntile) break;
        tile(integral_constant<int, 1>{}, sb);
        if (sb * NST + 2 >= ntile) break;
        tile(integral_constant<int, 2>{}, sb);
        if (sb * NST + 3 >= ntile) break;
        tile(integral_constant<int, 3>{}, sb);
    }
    wait_vm_lgkm0<0>();                              // loads past the chunk end and the stores are done
    if (fdst) store_state<D, C::SA, C::SB>(fdst, S, a0, b0, c, g);
}

// The 1 KiB piece filled by wave instruction gi (IPW per wave, NI pieces
// per tensor tile, RGN 16-row groups per tile): 16 rows (row0..) of the
// 32-element column block blk of the K (gi < NI) or V tile.  With ROPE the
// IPW pieces of a wave are consecutive column blocks of one row group, so the
// wave that loads column blocks 0 and 1 of a row group holds both halves of
// every rotary pair of those rows (dims i and i + 32 for d = 128; for d = 64
// dims i and i + 16 are both in block 0).
template <int NI, int IPW, int RGN, bool ROPE>
__device__ __forceinline__ void dma_piece(int gi, bool &isv, int &blk, int &row0) {
    isv = gi >= NI;
    const int x = isv ? gi - NI : gi;
    if constexpr (ROPE) {
        static_assert(NI % (IPW * RGN) == 0, "whole row groups per wave");
        const int wk = x / IPW, ii = x % IPW;
        blk = ii + IPW * (wk / RGN);
        row0 = 16 * (wk % RGN);
    } else {
        blk = x / RGN;
        row0 = 16 * (x % RGN);
    }
}

// Rotary-pair frequency setup of a lane that rotates K rows of a tile: the
// waves holding column block 0 of row group w (w < RGN) rotate rows
// 16 w + l / 4; the lane's 16-byte chunk is logical chunk lc of its row.
struct RopeK {
    bool on;        // this wave rotates K pieces
    int rowk;       // row within a tile
    int lc;         // logical 16-byte chunk (dims 8 lc .. 8 lc + 7 of block 0)
};

template <int D, int TJ>
__device__ __forceinline__ RopeK rope_k_lane(int w, int l) {
    RopeK r;
    r.on = w < TJ / 16;
    r.rowk = 16 * w + (l >> 2);
    r.lc = (int)((l & 3) ^ SubRows<TJ>::swz(r.rowk));
    return r;
}

// U_c = K_c^T V_c over a sub-chunk, with the K/V tiles staged through
// registers: each wave loads its 16-byte pieces of tile t + 2 into registers
// (buffer loads, rows past the sub-chunk end read as zeros) while tile t is
// summed, and writes tile t + 1 into the other LDS stage at the end of tile
// t.  Same LDS layout as the fused kernel's tiles.  Measured on MI355X,
// buffer-to-LDS loads alone stream at most ~6.3 TB/s and register loads
// ~7.3 TB/s; this kernel does little besides streaming, and staging through
// registers made it a little faster (about 1% on the 1M-token workload).
//
// With ROPE the K rows are rotated in registers before they go to LDS.
template <int D, int BLK, int NW, bool ROPE>
__global__ __launch_bounds__(NW * 64, 1024 / (NW * 64)) void k_summary_reg(KParams p) {
    using C = Cfg<bf16_t, D, BLK, NW>;
    constexpr int TJ = C::TJ;
    using LT = SubRows<TJ>;
    constexpr int RB = D * 2;                        // bytes per token row
    constexpr int TB = TJ * RB;                      // bytes of one tensor tile
    constexpr int SBY = 2 * TB;                      // stage: K tile then V tile
    constexpr int NI = TB / 1024;                    // 1 KiB pieces per tensor tile
    constexpr int IPW = 2 * NI / NW;                 // pieces per wave per tile
    static_assert((2 * NI) % NW == 0 && TB % 1024 == 0, "tile split");
    char *stages[2];
    Ring<2, SBY>::get(stages);
    const int h = blockIdx.y;
    const int gch = blockIdx.x;
    if (gch >= sub_off(p, p.nseq)) return;
    const int s = seq_of_sub(p, gch);
    const int64_t t0 = sub_first_token(p, s, gch);
    if (t0 < 0) return;                              // in the sequence's last chunk: not needed
    const Unit u = unit_of<D>(p, s, h);
    const int n = (int)min(u.len - t0, p.sub);       // tokens of this sub-chunk
    const int64_t cb = (u.base + t0 * D) * 2;
    const uint32_t nbytes = (uint32_t)n * RB;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const char *>(p.k) + cb, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const char *>(p.v) + cb, nbytes);

    const int w = wave_id(), l = lane_id(), c = l & 15, g = l >> 4;
    const int a0 = C::SA * (w % C::AW), b0 = C::SB * (w / C::AW);
    uint32_t ka_off[C::SA], vb_off[C::SB];
#pragma unroll
    for (int ia = 0; ia < C::SA; ++ia) ka_off[ia] = col_tile_off<TJ>(l, a0 + ia);
#pragma unroll
    for (int ib = 0; ib < C::SB; ++ib) vb_off[ib] = TB + col_tile_off<TJ>(l, b0 + ib);

    // piece gi = w * IPW + ii: 16 rows of one 32-element column block of the
    // K (gi < NI) or V tile; lane l brings row row0 + l / 4, physical 16-byte
    // chunk l % 4, and writes it at LDS byte dlo + 16 l of the stage
    uint32_t dvo[IPW], dlo[IPW];
    __amdgpu_buffer_rsrc_t drs[IPW];
#pragma unroll
    for (int ii = 0; ii < IPW; ++ii) {
        bool isv;
        int blk, row0;
        dma_piece<NI, IPW, TJ / 16, ROPE>(w * IPW + ii, isv, blk, row0);
        const int row = row0 + (l >> 2);
        dvo[ii] = (uint32_t)(row * RB + blk * 64 + (((l & 3) ^ LT::swz(row)) << 4));
        dlo[ii] = (isv ? TB : 0) + blk * LT::BLOCK + row0 * 64 + 16 * l;
        drs[ii] = isv ? rv : rk;
    }
    u32x4_t R0[IPW], R1[IPW];
    // rotary embedding of the K rows this lane brings (tile `tile`)
    [[maybe_unused]] const RopeK rk_lane = rope_k_lane<D, TJ>(w, l);
    [[maybe_unused]] RopeFreqs rf8{};
    [[maybe_unused]] int64_t pbase = 0;
    if constexpr (ROPE) {
        rf8 = rope_freqs(p.rope_base, p.rope_dims);
        pbase = (p.pos0 ? (int64_t)p.pos0[s] : 0) + t0;
    }
    auto rot = [&](u32x4_t (&R)[IPW], int tile) {
        if constexpr (ROPE) {
            if (rk_lane.on) {
                const double pos = (double)(pbase + (int64_t)tile * TJ + rk_lane.rowk);
                if constexpr (D == 128) {
                    rope_rot8(R[0], R[1], pos, rope_f(rk_lane.lc, rf8), rf8.rho);
                } else {
                    u32x4_t other;
#pragma unroll
                    for (int d = 0; d < 4; ++d)   // lane l ^ 2 holds chunk lc ^ 2 of the same row
                        other[d] = (uint32_t)__builtin_amdgcn_mov_dpp((int)R[0][d], 0x4E, 0xF, 0xF, false);
                    R[0] = rope_rot8_half(R[0], other, rk_lane.lc < 2, pos, rope_f(rk_lane.lc & 1, rf8), rf8.rho);
                }
            }
        }
    };
    auto load = [&](int tile, u32x4_t (&R)[IPW]) {
#pragma unroll
        for (int ii = 0; ii < IPW; ++ii)
            R[ii] = __builtin_amdgcn_raw_buffer_load_b128(drs[ii], (int)dvo[ii], tile * TB, 0);
    };
    auto put = [&](char *stage, const u32x4_t (&R)[IPW]) {
#pragma unroll
        for (int ii = 0; ii < IPW; ++ii) *reinterpret_cast<u32x4_t *>(stage + dlo[ii]) = R[ii];
    };

    f32x4_t S[C::SA][C::SB];
#pragma unroll
    for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
        for (int ib = 0; ib < C::SB; ++ib) S[ia][ib] = zero4();
    auto sum_tile = [&](const char *stage) {
        const char *ka[C::SA];
        const char *vb[C::SB];
#pragma unroll
        for (int ia = 0; ia < C::SA; ++ia) ka[ia] = stage + ka_off[ia];
#pragma unroll
        for (int ib = 0; ib < C::SB; ++ib) vb[ib] = stage + vb_off[ib];
        state_update_tr<TJ, C::SA, C::SB>(S, ka, vb);
    };

    const int ntile = (n + TJ - 1) / TJ;
    load(0, R0);
    load(1, R1);
    rot(R0, 0);
    put(stages[0], R0);
    wait_vm_lgkm0<63>();                             // own LDS writes done
    wg_barrier();
    for (int t = 0; t < ntile; t += 2) {
        load(t + 2, R0);                             // past the end: zeros, never used
        sum_tile(stages[0]);
        rot(R1, t + 1);
        put(stages[1], R1);                          // tile t + 1 (stage 1 was last read in tile t - 1)
        wait_vm_lgkm0<63>();
        wg_barrier();
        if (t + 1 < ntile) {
            load(t + 3, R1);
            sum_tile(stages[1]);
            rot(R0, t + 2);
            put(stages[0], R0);                      // tile t + 2
            wait_vm_lgkm0<63>();
            wg_barrier();
        }
    }
    wait_vm_lgkm0<0>();
    float *dst = p.states + ((int64_t)h * p.nsub_ub + gch) * (D * D);
#pragma unroll
    for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
        for (int ib = 0; ib < C::SB; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[((a0 + ia) * 16 + 4 * g + r) * D + (b0 + ib) * 16 + c] = S[ia][ib][r];
}

// Which 32-element groups [lo(jt), hi(jt)) of the next block's Q a wave
// requests in tile jt of a block with TPB tiles (none in the last tile), and
// how many loads that is (n(-1) = 0: the tile before a block's first).
template <int TPB, int KC, int NSW>
struct QSplit {
    static constexpr int lo(int jt) {
        return TPB == 4 ? (jt == 0 ? 0 : jt == 1 ? KC / 4 : jt == 2 ? KC / 2 : KC) : (TPB == 2 && jt == 0 ? 0 : KC);
    }
    static constexpr int hi(int jt) {
        return TPB == 4 ? (jt == 0 ? KC / 4 : jt == 1 ? KC / 2 : KC) : (TPB == 2 && jt == 0 ? KC : KC);
    }
    static constexpr int n(int jt) { return jt < 0 ? 0 : NSW * (hi(jt) - lo(jt)); }
};

// Per chunk: walk the blocks carrying S; per block O^T = S^T Q^T + V^T P^T
// with P = mask(Q K^T), then S += K^T V.
//
// K and V stream through a 4-stage LDS ring in TJ = 64-token tiles, loaded
// by buffer loads straight into LDS; tile t + LA is requested while tile t is
// used.  The launcher takes LA = 2 (the fourth stage holds the tile before)
// except for chunks of kLongChunkTokens or more, where LA = 3 (the stage of
// tile t - 1, released by the barrier that ends it).
// The four tiles of a ring cycle (a "super-block" of 256 tokens, one
// or more whole blocks) are separate compile-time copies of the tile body, so
// a tile's stage, its place in its block and its wait counts are constants.
// All global accesses go through buffer resources that end at the chunk end:
// rows past it load as zeros (they add nothing to any product) and stores to
// them are dropped, so a final partial block or super-block is processed as a
// whole one.
//
// Vector-memory order and waits.  The ring stages are separate LDS arrays,
// so the compiler tracks each DMA by its destination and itself waits exactly
// for the loads a read needs (DMA, Q); O stores are issued from inline asm and
// stay outside its bookkeeping, which would otherwise treat loads and stores
// as unordered.  vmcnt counts both; loads complete in issue order but stores
// may complete ahead of older loads, so each explicit wait (the one before a
// barrier, which other waves rely on) bounds the loads younger than the one
// it needs:
//   the next block's Q is loaded over the block's tiles, each part at the
//   top of a tile ahead of its DMA;
//   tile not ending a block: DMA(t+LA) at its top; at its end DMA(t+1) must
//   have landed; younger are DMA(t+2 .. t+LA) and the Q loads of the LA-1
//   tiles up to this one;
//   tile ending a block: all of the next Q and DMA(t+1) must have landed;
//   younger is DMA(t+2 .. t+LA-1); then it requests DMA(t+LA);
//   a wave stores its O after the wait of the last tile that holds keys of
//   its rows (O is final there), so the stores spread over the block and
//   complete during the following tile.
// With one tile per block the next Q is loaded after the tile's scores and
// the tile waits for every load.
//
// With ROPE, q and k are rotated on the way in: each block's Q in registers
// once its loads have landed, each K tile in LDS by the waves that loaded
// column blocks 0 and 1 of its row groups, right after their own wait for
// that tile (before the barrier that publishes it).
template <int D, int BLK, int NW, int TJ, int NST, int LA, bool ROPE>
__global__ __launch_bounds__(NW * 64, 1) void k_fused_dma(KParams p) {
    using T = bf16_t;
    using C = Cfg<T, D, BLK, NW>;
    using LT = SubRows<TJ>;                          // K / V tiles
    using LS = SubRows<D>;                           // state copy S^T (rows = value dim)
    static_assert(LA >= 1 && LA < NST, "tiles requested ahead of the one in use");
    constexpr int TPB = BLK / TJ;                    // tiles per block
    constexpr int RB = D * 2;                        // bytes per token row
    constexpr int TB = TJ * RB;                      // bytes of one tensor tile
    constexpr int SBY = 2 * TB;                      // stage: K tile then V tile
    constexpr int NI = TB / 1024;                    // 1 KiB DMA instructions per tensor tile
    constexpr int IPW = 2 * NI / NW;                 // DMA instructions per wave per tile
    constexpr int QL = C::NSW * C::KC;               // Q loads per wave per block
    // The next block's Q is requested over the tiles of a block, a few
    // fragments per tile ahead of that tile's DMA: 32-element groups
    // [qlo(jt), qhi(jt)) in tile jt (none in the last tile; with one tile per
    // block Q is instead reloaded after that tile's scores).
    using QS = QSplit<TPB, C::KC, C::NSW>;
    static_assert(NST % TPB == 0 && (2 * NI) % NW == 0 && TB % 1024 == 0, "tile split");
    static_assert(C::NCT % 2 == 0, "column tiles are stored in pairs");
    __shared__ __attribute__((aligned(16))) char st[C::ST_BYTES];
    char *stages[NST];
    Ring<NST, SBY>::get(stages);

    int h, s;
    int64_t gch;
    if (!chunk_of_block(p, h, gch, s)) return;
    const Unit u = unit_of<D>(p, s, h);
    const int cl = (int)(gch - chunk_off(p, s));
    const int64_t t0 = (int64_t)cl * p.chunk;
    const int n = (int)min(u.len - t0, p.chunk);     // tokens of this chunk
    const int64_t cb = (u.base + t0 * D) * 2;        // byte offset of its first row
    const uint32_t nbytes = (uint32_t)n * RB;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const char *>(p.q) + cb, nbytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const char *>(p.k) + cb, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const char *>(p.v) + cb, nbytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<char *>(p.o) + cb, nbytes);

    const int w = wave_id(), l = lane_id(), c = l & 15, g = l >> 4;
    const int a0 = C::SA * (w % C::AW), b0 = C::SB * (w / C::AW);
    const int ct0 = col_tile0<BLK, NW, C::NCT>(w);
    const int nblk = (n + BLK - 1) / BLK;
    const int nsb = (nblk * TPB + NST - 1) / NST;    // super-blocks

    // ---- lane-constant LDS offsets
    const uint32_t row8 = LT::row8_base(c, g);       // == LS::row8_base(c, g)
    uint32_t ka_off[C::SA], vb_off[C::SB];
#pragma unroll
    for (int ia = 0; ia < C::SA; ++ia) ka_off[ia] = col_tile_off<TJ>(l, a0 + ia);
#pragma unroll
    for (int ib = 0; ib < C::SB; ++ib) vb_off[ib] = TB + col_tile_off<TJ>(l, b0 + ib);
    const uint32_t vpv_off = TB + col_tile_off<TJ>(l, ct0);       // ct0 is even
    const int par_step = (int)col_tile_off<TJ>(l, 1) - (int)col_tile_off<TJ>(l, 0);

    // ---- DMA: wave instruction gi = w * IPW + ii fills 16 rows (row0..) of
    // one 32-element column block of the K (gi < NI) or V tile; lane l brings
    // row row0 + l / 4, physical 16-byte chunk l % 4.
    uint32_t dvo[IPW], dlo[IPW];
    __amdgpu_buffer_rsrc_t drs[IPW];
#pragma unroll
    for (int ii = 0; ii < IPW; ++ii) {
        bool isv;
        int blk, row0;
        dma_piece<NI, IPW, TJ / 16, ROPE>(w * IPW + ii, isv, blk, row0);
        const int row = row0 + (l >> 2);
        dvo[ii] = (uint32_t)(row * RB + blk * 64 + (((l & 3) ^ LT::swz(row)) << 4));
        dlo[ii] = (isv ? TB : 0) + blk * LT::BLOCK + row0 * 64;
        drs[ii] = isv ? rv : rk;
    }
    auto issue = [&](int tile, char *stage) {
#pragma unroll
        for (int ii = 0; ii < IPW; ++ii)
            dma_lds16(drs[ii], stage + dlo[ii], dvo[ii], (uint32_t)(tile * TB));
    };

    // ---- Q rows of the wave's slabs: lane (c, g) loads row 16 slab + c,
    // elements 8g..8g+7 of each 32-element group kc
    uint32_t qvo[C::NSW], ovo[C::NSW];
    // O store m writes columns 16 (ct0 + 2m) + 4g .. +7 (even g) or
    // 16 (ct0 + 2m + 1) + 4 (g - 1) .. +7 (odd g): 64 m bytes further on
    auto o_off = [&](int si, int cc, int gg) {
        const int r = 16 * slab_of<BLK, NW>(w, si) + cc;
        return (uint32_t)(r * RB + 2 * ((gg & 1) ? 16 * (ct0 + 1) + 4 * (gg - 1) : 16 * ct0 + 4 * gg));
    };
#pragma unroll
    for (int si = 0; si < C::NSW; ++si) {
        const int r = 16 * slab_of<BLK, NW>(w, si) + c;
        qvo[si] = (uint32_t)(r * RB + g * 16);
        ovo[si] = o_off(si, c, g);
    }
    // Q of the current block, and of the next one (requested a tile early
    // when blocks have two or more tiles)
    Frag<T> Q[C::NSW][C::KC], Qn[C::NSW][C::KC];
    auto load_q = [&](Frag<T> (&dst)[C::NSW][C::KC], int row0, int k0, int k1) {
#pragma unroll
        for (int si = 0; si < C::NSW; ++si)
#pragma unroll
            for (int kc = 0; kc < C::KC; ++kc)
                if (kc >= k0 && kc < k1)
                    dst[si][kc].u = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)qvo[si] + kc * 64, row0 * RB, 0);
    };
    // Tile of a block after which the wave's O is final and its Q unused:
    // the last tile holding keys of its last row slab.  The wave stores its O
    // there, so the stores of a block spread over its tiles.
    int smax = 0;
#pragma unroll
    for (int si = 0; si < C::NSW; ++si) smax = max(smax, slab_of<BLK, NW>(w, si));
    const int jl = min(TPB - 1, (16 * smax + 15) / TJ);

    // state copy S^T: lane writes row b = 16(b0+ib) + c, elements 16(a0+ia) + 4g .. +3
    auto write_state = [&](const f32x4_t (&Sx)[C::SA][C::SB]) {
        const int lf = lane_id_fresh(), cf = lf & 15, gf = lf >> 4;
#pragma unroll
        for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
            for (int ib = 0; ib < C::SB; ++ib)
                lds_store8(st + LS::off((b0 + ib) * 16 + cf, (a0 + ia) * 16 + 4 * gf),
                           u32x2_t{pack_bf16x2(Sx[ia][ib][0], Sx[ia][ib][1]), pack_bf16x2(Sx[ia][ib][2], Sx[ia][ib][3])});
    };

    // ---- rotary embedding: K rows of tile `tile` in its ring stage (by the
    // lanes that loaded them), the Q rows of the block starting at token tq
    [[maybe_unused]] const RopeK rk_lane = rope_k_lane<D, TJ>(w, l);
    [[maybe_unused]] RopeFreqs rf8{};
    [[maybe_unused]] int64_t pbase = 0;
    if constexpr (ROPE) {
        rf8 = rope_freqs(p.rope_base, p.rope_dims);
        pbase = (p.pos0 ? (int64_t)p.pos0[s] : 0) + t0;
    }
    // (lane-derived values are taken from lane_id_fresh() so that the pair
    // frequencies are recomputed at each use rather than held in registers)
    auto rot_k = [&](char *stage, int tile) {
        if constexpr (ROPE) {
            if (rk_lane.on) {
                const int lf = (int)lane_id_fresh();
                const RopeK rf = rope_k_lane<D, TJ>(w, lf);
                const double pos = (double)(pbase + (int64_t)tile * TJ + rf.rowk);
                u32x4_t *a = reinterpret_cast<u32x4_t *>(stage + dlo[0] + 16 * lf);
                if constexpr (D == 128) {
                    // the lane's chunk of column block 0 and, a block further, its partner
                    u32x4_t *b = reinterpret_cast<u32x4_t *>(stage + dlo[0] + LT::BLOCK + 16 * lf);
                    u32x4_t x = *a, y = *b;
                    rope_rot8(x, y, pos, rope_f(rf.lc, rf8), rf8.rho);
                    *a = x;
                    *b = y;
                } else {
                    // partner: chunk lc ^ 2 of the same row, brought by lane l ^ 2
                    const u32x4_t x = *a;
                    const u32x4_t y = *reinterpret_cast<const u32x4_t *>(stage + dlo[0] + 16 * (lf ^ 2));
                    *a = rope_rot8_half(x, y, rf.lc < 2, pos, rope_f(rf.lc & 1, rf8), rf8.rho);
                }
            }
        }
    };
    auto rot_q = [&](Frag<T> (&Q)[C::NSW][C::KC], int tq) {
        if constexpr (ROPE) {
            const int lf = lane_id_fresh(), cf = lf & 15, gf = lf >> 4;
#pragma unroll
            for (int si = 0; si < C::NSW; ++si) {
                const double pos = (double)(pbase + tq + 16 * slab_of<BLK, NW>(w, si) + cf);
                if constexpr (D == 128) {
                    // dims 8g .. 8g+7 (group 0) pair with dims 32 + 8g .. (group 1)
                    rope_rot8(Q[si][0].u, Q[si][1].u, pos, rope_f(gf, rf8), rf8.rho);
                } else {
                    // dims 8g .. 8g+7 of group 0 pair with lane l ^ 32's (g ^ 2)
                    u32x4_t other;
#pragma unroll
                    for (int d = 0; d < 4; ++d) other[d] = (uint32_t)__shfl_xor((int)Q[si][0].u[d], 32);
                    Q[si][0].u = rope_rot8_half(Q[si][0].u, other, gf < 2, pos, rope_f(gf & 1, rf8), rf8.rho);
                }
            }
        }
    };

    // ---- prologue: the first block's Q, tile 0 (and tile 1 when three are
    // kept in flight), the state at the chunk start (exclusive prefix from
    // the scan; zero for a sequence's first chunk); tile LA - 1 stays in flight
    f32x4_t S[C::SA][C::SB];
    load_q(Q, 0, 0, C::KC);
    issue(0, stages[0]);
    if constexpr (LA >= 3) issue(1, stages[1]);
    float *const fdst = final_state_dst<D>(p, s, h, gch);
    const float *const src = chunk_start_state<D>(p, s, h, cl);
    const bool zs = src == nullptr;
    {
#pragma unroll
        for (int ia = 0; ia < C::SA; ++ia)
#pragma unroll
            for (int ib = 0; ib < C::SB; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[ia][ib][r] = src ? src[((a0 + ia) * 16 + 4 * g + r) * D + (b0 + ib) * 16 + c] : 0.f;
        write_state(S);
    }
    wait_vm_lgkm0<0>();
    if constexpr (ROPE) {
        rot_q(Q, 0);
        rot_k(stages[0], 0);
    }
    if constexpr (LA >= 2) issue(LA - 1, stages[LA - 1]);
    if constexpr (ROPE) wait_vm_lgkm0<63>();         // the rotated tile is written
    wg_barrier();

    f32x4_t O[C::NSW][C::NCT];
    // ---- store the O of block bi.  Lane (c, g) holds row 16 slab + c, columns
    // 16 ct + 4g .. +3 of every column tile ct.  Lanes 16 apart (g, g^1) swap
    // one 8-byte half so that each stores 16 contiguous bytes: the even-g lane
    // columns 16 ct + 4g .. +7 of the even tile of a pair, the odd-g lane those
    // of the odd tile.  Four lanes cover 64 contiguous bytes of a row.
    auto store_o = [&](int bi) {
#pragma unroll
        for (int si = 0; si < C::NSW; ++si) {
            // (with ROPE recomputed here, which keeps a register free)
            const int lf = ROPE ? (int)lane_id_fresh() : 0;
            const int vo = (int)(ROPE ? o_off(si, lf & 15, lf >> 4) : ovo[si]) + bi * BLK * RB;
#pragma unroll
            for (int m = 0; m < C::NCT / 2; ++m) {
                const uint32_t e0 = pack_bf16x2(O[si][2 * m][0], O[si][2 * m][1]);
                const uint32_t e1 = pack_bf16x2(O[si][2 * m][2], O[si][2 * m][3]);
                const uint32_t o0 = pack_bf16x2(O[si][2 * m + 1][0], O[si][2 * m + 1][1]);
                const uint32_t o1 = pack_bf16x2(O[si][2 * m + 1][2], O[si][2 * m + 1][3]);
                // v_permlane16_swap exchanges the odd 16-lane rows of its first
                // operand with the even rows of its second: an even-g lane keeps
                // its even-tile words and gets its odd-g partner's, an odd-g lane
                // gets its partner's odd-tile words and keeps its own
                const auto x0 = __builtin_amdgcn_permlane16_swap(e0, o0, false, false);
                const auto x1 = __builtin_amdgcn_permlane16_swap(e1, o1, false, false);
                store16(ro, (uint32_t)(vo + m * 64), u32x4_t{x0[0], x1[0], x0[1], x1[1]});
            }
        }
    };

    using std::integral_constant;

    auto tile = [&](auto J_c, int sb) {
        constexpr int J = decltype(J_c)::value;     // tile within the super-block = ring stage
        static_assert(J < NST, "one tile per ring stage");
        constexpr int jt = J % TPB;                  // tile within its block
        constexpr bool first = jt == 0, last = jt == TPB - 1;
        const int t = sb * NST + J;
        const int bi = sb * (NST / TPB) + J / TPB;
        const int tb = bi * BLK;                     // block's first token (chunk-relative)
        const bool more = bi + 1 < nblk;
        if constexpr (QS::n(jt) > 0) load_q(Qn, tb + BLK, QS::lo(jt), QS::hi(jt));
        // DMA(t + LA) at the top of the tile (with two or more tiles in
        // flight a block's last tile requests it after its wait instead)
        if constexpr (!last || LA == 1) issue(t + LA, stages[(J + LA) % NST]);
        const char *stage = stages[J];
        const char *krow = stage + row8;             // K rows (b128 reads)
        const char *vcol = stage + vpv_off;          // V columns of tile ct0 (tr reads)

        // a chunk that starts from zero has Q S = 0 in its first block
        bool zero_s = false;
        if constexpr (first && J < TPB) zero_s = zs && sb == 0;
        // (one slab per wave: a slab starting past the chunk end has no output)
        if constexpr (first && C::NSW == 1) zero_s = zero_s || 16 * slab_of<BLK, NW>(w, 0) >= n - tb;
        if (zero_s) {
#pragma unroll
            for (int si = 0; si < C::NSW; ++si)
#pragma unroll
                for (int ct = 0; ct < C::NCT; ++ct) O[si][ct] = zero4();
        } else if constexpr (first) {
            // ---- inter-block right product with the block-start state
            const char *srow = st + row8 + ct0 * 16 * 64;
#pragma unroll
            for (int ct = 0; ct < C::NCT; ++ct) {
                // all KC fragments of the column tile are requested before the
                // first product, so one LDS latency covers KC products
                Frag<T> A[C::KC];
#pragma unroll
                for (int kc = 0; kc < C::KC; ++kc) A[kc] = ld_row8<T>(srow + kc * LS::BLOCK + ct * 16 * 64);
                hold(A);
#pragma unroll
                for (int si = 0; si < C::NSW; ++si) O[si][ct] = zero4();
#pragma unroll
                for (int kc = 0; kc < C::KC; ++kc)
#pragma unroll
                    for (int si = 0; si < C::NSW; ++si) mma(O[si][ct], A[kc], Q[si][kc]);
                sched_fence();
            }
        }
        if constexpr (ROPE && last && TPB > 1) {
            // the rotated dims of the next block's Q were requested in the
            // block's earlier tiles: rotate them while this tile's products run
            if (more) rot_q(Qn, tb + BLK);
        }

        // ---- intra-block left product for this K/V tile
#pragma unroll
        for (int jg = 0; jg < TJ / 32; ++jg) {
            constexpr int jt_ = jt;
            const int jb = jt_ * TJ + jg * 32;       // block-local first token of the group
            f32x4_t P[C::NSW][2];
            bool need[C::NSW], need1[C::NSW];
#pragma unroll
            for (int si = 0; si < C::NSW; ++si) {
                const int i0 = 16 * slab_of<BLK, NW>(w, si);
                // last key the slab sees: keys past the chunk end add nothing,
                // and a slab starting past it has no output (-1: skip all)
                const int left = n - tb;
                const int kmax = i0 < left ? min(i0 + 15, left - 1) : -1;
                need[si] = jb <= kmax;
                need1[si] = jb + 16 <= kmax;
                P[si][0] = zero4();
                P[si][1] = zero4();
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                bool any = false;
#pragma unroll
                for (int si = 0; si < C::NSW; ++si) any |= hh ? need1[si] : need[si];
                if (!any) continue;
                Frag<T> A[C::KC];
#pragma unroll
                for (int kc = 0; kc < C::KC; ++kc) A[kc] = ld_row8<T>(krow + kc * LT::BLOCK + (jg * 32 + 16 * hh) * 64);
                hold(A);
#pragma unroll
                for (int kc = 0; kc < C::KC; ++kc)
#pragma unroll
                    for (int si = 0; si < C::NSW; ++si)
                        if (hh ? need1[si] : need[si]) mma(P[si][hh], A[kc], Q[si][kc]);
                sched_fence();
            }
            Frag<T> PF[C::NSW];
#pragma unroll
            for (int si = 0; si < C::NSW; ++si) {
                const int i0 = 16 * slab_of<BLK, NW>(w, si);
                const int i = i0 + c;
                if (need[si] && jb + 31 > i0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (jb + 4 * g + r > i) P[si][0][r] = 0.f;
                        if (jb + 16 + 4 * g + r > i) P[si][1][r] = 0.f;
                    }
                }
                PF[si] = frag_from_f32(P[si][0], P[si][1], T{});
            }
            bool anyg = false;
#pragma unroll
            for (int si = 0; si < C::NSW; ++si) anyg |= need[si];
            if (anyg) {
                // batches of PB column tiles: their V fragments are requested
                // together, then PB products
                constexpr int PB = C::NCT < 4 ? C::NCT : 4;
#pragma unroll
                for (int cb = 0; cb < C::NCT; cb += PB) {
                    Frag<T> A[PB];
#pragma unroll
                    for (int b = 0; b < PB; ++b) {
                        // column tile ct0 + ct: parity ct & 1 (ct0 even), block (ct0 + ct) / 2
                        const int ct = cb + b;
                        A[b] = ld_cols8(vcol + (ct >> 1) * LT::BLOCK + jg * 32 * 64 + (ct & 1 ? par_step : 0));
                    }
                    hold(A);
#pragma unroll
                    for (int b = 0; b < PB; ++b)
#pragma unroll
                        for (int si = 0; si < C::NSW; ++si)
                            if (need[si]) mma(O[si][cb + b], A[b], PF[si]);
                    sched_fence();
                }
            }
        }

        // rotate the next tile's keys while the other waves are still on this
        // tile's products; the barrier at the end of the tile publishes them.
        // Not in a block's last tile: there the next tile's DMA is the newest
        // request, and waiting for it here would drain the queue, so the
        // rotation follows the tile's own wait instead.
        if constexpr (ROPE && !last) rot_k(stages[(J + 1) % NST], t + 1);

        const char *ka[C::SA];
        const char *vbs[C::SB];
#pragma unroll
        for (int ia = 0; ia < C::SA; ++ia) ka[ia] = stage + ka_off[ia];
#pragma unroll
        for (int ib = 0; ib < C::SB; ++ib) vbs[ib] = stage + vb_off[ib];

        if constexpr (last) {
            if constexpr (TPB == 1) load_q(Q, tb + BLK, 0, C::KC);   // this block's Q is dead after its scores
            if ((more || fdst) && jt * TJ < n - tb) state_update_tr<TJ, C::SA, C::SB>(S, ka, vbs);
            if (more) {
                if constexpr (first) {               // one-tile blocks: the state copy was read in this tile
                    wait_vm_lgkm0<63>();
                    wg_barrier();
                }
                write_state(S);
            }
            // the next block's Q and DMA(t+1) have landed; younger is
            // DMA(t+2 .. t+LA-1) (with one tile per block Q itself was
            // reloaded in this tile and everything is waited for)
            if constexpr (TPB == 1) {
                wait_vm_lgkm0<0>();
                if constexpr (ROPE) {
                    if (more) rot_q(Q, tb + BLK);        // loaded in this tile
                }
            } else {
                wait_vm_lgkm0<(LA >= 2 ? (LA - 2) * IPW : 0)>();
#pragma unroll
                for (int si = 0; si < C::NSW; ++si)
#pragma unroll
                    for (int kc = 0; kc < C::KC; ++kc) Q[si][kc] = Qn[si][kc];
            }
            if constexpr (ROPE) rot_k(stages[(J + 1) % NST], t + 1);
            if constexpr (LA > 1) issue(t + LA, stages[(J + LA) % NST]);
            if constexpr (ROPE) wait_vm_lgkm0<63>();     // the rotated tile is written
        } else {
            if ((more || fdst) && jt * TJ < n - tb) state_update_tr<TJ, C::SA, C::SB>(S, ka, vbs);
            // DMA(t+1) has landed; younger are DMA(t+2 .. t+LA) and the Q
            // loads of the LA-1 tiles up to this one
            wait_vm_lgkm0<(LA - 1) * IPW + (LA >= 2 ? QS::n(jt) : 0) + (LA >= 3 ? QS::n(jt - 1) : 0)>();
        }
        if (jt == jl) store_o(bi);
        wg_barrier();
    };

    // Tiles past the chunk's last token hold only zeros: with blocks of two
    // or more tiles the walk stops after the last tile with tokens
    // (wave-uniform).  Every wave with rows in the chunk has stored its O by
    // then, since a 16-row slab never straddles a tile; the rest of the block
    // would only add zeros to the state.  (With one tile per block the
    // compiler drains the whole load queue at such exits, so that walk keeps
    // its padding blocks.)
    static_assert(NST == 4, "ring stages");
    const int ntile = TPB > 1 ? (n + TJ - 1) / TJ : nsb * NST;
    for (int sb = 0; sb < nsb; ++sb) {
        tile(integral_constant<int, 0>{}, sb);
        if (TPB > 1 && sb * NST + 1 >= ntile) break;
        tile(integral_constant<int, 1>{}, sb);
        if (TPB > 1 && sb * NST + 2 >= ntile) break;
        tile(integral_constant<int, 2>{}, sb);
        if (TPB > 1 && sb * NST + 3 >= ntile) break;
        tile(integral_constant<int, 3>{}, sb);
    }
    wait_vm_lgkm0<0>();                              // DMA past the chunk end and the stores are done
    if (fdst) {
        const int lf = lane_id_fresh();
        store_state<D, C::SA, C::SB>(fdst, S, a0, b0, lf & 15, lf >> 4);
    }
}

// -------------------------------------------------------------- host side

// Waves per workgroup of the bf16 fused kernel: sixteen (one 16-row slab
// each, slabs of blocks of 128 split by output columns over two waves)
// except for 64-token blocks, where the column split would make four waves
// recompute each slab's scores.  Measured on MI355X at 4 x 64 heads x 8192
// tokens: 16 waves are 7-11% faster than 8 for d = 64 (blocks of 128 and
// 256) and d = 128 (blocks of 128), and 23% slower for d = 128, blocks of 64.
constexpr int fused_waves(int D, int BLK) { return BLK == 64 ? 8 : 16; }

// K/V tiles in flight in the bf16 fused kernel: three for chunks of this many
// tokens or more, two otherwise.  Alternating in one session on MI355X, three
// were 4-6% faster at 64 heads x 1M tokens (chunks of 262,144), neutral at
// chunks of 32,768-65,536 and 0.5-2.7% slower on the MiniMax layer (chunks of
// 8,192) and on packed sequences of 64-2,047 tokens; outputs bit-identical.
// The rotary instance measured the same with either at 1M tokens (its
// rotation work is what sets its pace there) and keeps two.
constexpr int64_t kLongChunkTokens = 131072;

template <typename T, int D, int BLK, bool ROPE>
static hipError_t launch_typed(const KParams &kp, const FwdPlan &plan, hipStream_t st, void *const *ev) {
    auto mark = [&](int i) {
        if (ev && ev[i]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[i]), st);
    };
    const dim3 gchunks((unsigned)plan.nchunk_ub, (unsigned)kp.heads);
    const dim3 gsubs((unsigned)plan.nsub_ub, (unsigned)kp.heads);
    mark(0);
    // packed input: the offset tables from cu_seqlens (dense input needs none),
    // and the final states of sequences with no tokens (every dense sequence
    // has tokens here: a call with none never reaches the kernels)
    if (kp.cu) {
        hipLaunchKernelGGL(k_prep, dim3(1), dim3(kPrepThreads), 0, st, kp);
        if (kp.s_final && !kp.slots)
            hipLaunchKernelGGL(k_state_empty<D>, dim3(kp.nseq, kp.heads), dim3(256), 0, st, kp);
    }
    mark(1);
    // Every chunk but the first of its sequence needs the exclusive prefix of
    // the chunk summaries before it; with one chunk per sequence there is none.
    if (!plan.single_chunk) {
        if constexpr (sizeof(T) == 2)
            hipLaunchKernelGGL((k_summary_reg<D, BLK, 8, ROPE>), gsubs, dim3(512), 0, st, kp);
        else
            hipLaunchKernelGGL((k_summary<T, D, BLK, ROPE>), gsubs, dim3(512), 0, st, kp);
    }
    mark(2);
    if (!plan.single_chunk) {
        const dim3 gtiles((unsigned)plan.ntile_ub, (D * D) / kScanThreads, (unsigned)kp.heads);
        if (plan.scan_tiles) {
            hipLaunchKernelGGL(k_scan_reduce<D>, gtiles, dim3(kScanThreads), 0, st, kp);
            hipLaunchKernelGGL(k_scan_tiles<D>, gtiles, dim3(kScanThreads), 0, st, kp);
        }
        hipLaunchKernelGGL(k_scan_apply<D>, gtiles, dim3(kScanThreads), 0, st, kp, plan.scan_tiles ? 1 : 0);
    }
    mark(3);
    if constexpr (sizeof(T) == 2) {
        constexpr int NWF = fused_waves(D, BLK);
        if constexpr (BLK >= 128 && !ROPE) {
            if (plan.chunk >= kLongChunkTokens) {
                hipLaunchKernelGGL((k_fused_dma<D, BLK, NWF, 64, 4, 3, ROPE>), gchunks, dim3(NWF * 64), 0, st,
                                   kp);
                mark(4);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((k_fused_dma<D, BLK, NWF, 64, 4, 2, ROPE>), gchunks, dim3(NWF * 64), 0, st, kp);
    }
    else if constexpr (D == 64 && !ROPE)
        hipLaunchKernelGGL((k_fused_ring<BLK>), gchunks, dim3(512), 0, st, kp);
    else
        hipLaunchKernelGGL((k_fused<T, D, BLK, ROPE>), gchunks, dim3(512), 0, st, kp);
    mark(4);
    return hipGetLastError();
}

template <typename T, int D, bool ROPE = false>
static hipError_t launch_blk(const KParams &kp, const FwdPlan &plan, int blk, hipStream_t st,
                             void *const *ev) {
    switch (blk) {
        case 64: return launch_typed<T, D, 64, ROPE>(kp, plan, st, ev);
        case 128: return launch_typed<T, D, 128, ROPE>(kp, plan, st, ev);
        default: return launch_typed<T, D, 256, ROPE>(kp, plan, st, ev);
    }
}

// Compute units of the current device, queried once per device and cached
// (the only state the library keeps).  A partitioned GPU reports its own
// share, so the plan balances chunks over the CUs that actually run them.
int device_cu_count() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cached[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

int read_cu_error(const FwdArgs &a, void *stream, int *flag) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int32_t h = 0;
    hipError_t e = hipMemcpyAsync(&h, a.workspace + a.plan.off_err, sizeof(h), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    *flag = h;
    return (int)e;
}

int launch_state_empty(const float *s_init, float *s_final, int nseq, int heads, int head_dim,
                       void *stream) {
    KParams kp{};
    kp.seq_len = 0;
    kp.cu = nullptr;
    kp.nseq = nseq;
    kp.heads = heads;
    kp.s_init = s_init;
    kp.s_final = s_final;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (head_dim == 64) hipLaunchKernelGGL(k_state_empty<64>, dim3(nseq, heads), dim3(256), 0, st, kp);
    else hipLaunchKernelGGL(k_state_empty<128>, dim3(nseq, heads), dim3(256), 0, st, kp);
    return (int)hipGetLastError();
}

int launch_fwd(const FwdArgs &a, void *stream, void *const *events) {
    KParams kp;
    kp.q = a.q; kp.k = a.k; kp.v = a.v; kp.o = a.o;
    kp.cu = a.cu_seqlens;
    kp.chunk_off = reinterpret_cast<int32_t *>(a.workspace + a.plan.off_chunk_off);
    kp.sub_off = reinterpret_cast<int32_t *>(a.workspace + a.plan.off_sub_off);
    kp.perm = a.cu_seqlens ? reinterpret_cast<int32_t *>(a.workspace + a.plan.off_perm) : nullptr;
    kp.rank_off = a.cu_seqlens ? reinterpret_cast<int32_t *>(a.workspace + a.plan.off_rank_off) : nullptr;
    kp.slot_tab = a.cu_seqlens ? reinterpret_cast<int32_t *>(a.workspace + a.plan.off_slot_tab) : nullptr;
    kp.tile_off = reinterpret_cast<int32_t *>(a.workspace + a.plan.off_tile_off);
    kp.err = a.cu_seqlens ? reinterpret_cast<int32_t *>(a.workspace + a.plan.off_err) : nullptr;
    kp.states = reinterpret_cast<float *>(a.workspace + a.plan.off_states);
    kp.tilesum = reinterpret_cast<float *>(a.workspace + a.plan.off_tilesum);
    kp.seq_len = a.seq_len;
    kp.chunk = a.plan.chunk;
    kp.sub = a.plan.sub;
    kp.nchunk_ub = a.plan.nchunk_ub;
    kp.nsub_ub = a.plan.nsub_ub;
    kp.ntile_ub = a.plan.ntile_ub;
    kp.nseq = a.nseq;
    kp.heads = a.heads;
    kp.group = a.plan.scan_group;
    if (!a.cu_seqlens) {                             // dense: the same counts for every sequence
        const int64_t C = a.plan.chunk, Cs = a.plan.sub, G = a.plan.scan_group;
        kp.cps = (a.seq_len + C - 1) / C;
        kp.nsps = kp.cps >= 2 ? (kp.cps - 1) * (C / Cs) + 1 : 0;
        kp.tps = (kp.nsps + G - 1) / G;
    } else {
        kp.cps = kp.nsps = kp.tps = 0;
    }
    kp.s_init = a.s_init;
    kp.s_final = a.s_final;
    kp.slots = a.slots;
    kp.nslots = a.nslots;
    kp.init_mode = (a.s_init == nullptr && a.slots == nullptr) ? 0 : (a.plan.single_chunk ? 2 : 1);
    kp.pos0 = a.pos0;
    kp.rope_base = a.rope_base;
    kp.rope_dims = a.rope_dims;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (a.rope_dims > 0) {
        // rope_dims == head_dim / 2 (checked by the caller)
        if (a.dtype == 0)
            e = a.head_dim == 64 ? launch_blk<bf16_t, 64, true>(kp, a.plan, a.block_size, st, events)
                                 : launch_blk<bf16_t, 128, true>(kp, a.plan, a.block_size, st, events);
        else
            e = a.head_dim == 64 ? launch_blk<float, 64, true>(kp, a.plan, a.block_size, st, events)
                                 : launch_blk<float, 128, true>(kp, a.plan, a.block_size, st, events);
    } else if (a.dtype == 0) {
        e = a.head_dim == 64 ? launch_blk<bf16_t, 64>(kp, a.plan, a.block_size, st, events)
                             : launch_blk<bf16_t, 128>(kp, a.plan, a.block_size, st, events);
    } else {
        e = a.head_dim == 64 ? launch_blk<float, 64>(kp, a.plan, a.block_size, st, events)
                             : launch_blk<float, 128>(kp, a.plan, a.block_size, st, events);
    }
    return (int)e;
}

}  // namespace la
