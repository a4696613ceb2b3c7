// S1 + S2: int8 indexer scoring on the matrix cores and an exact radix top-k.
//
// Scoring ("What moved the number from 19.4 to 122.9 tokens a second?", Introducing Kiln: dedicated
// scoring and top-k kernels over a separate key cache).  score[p] = sum_h relu(q_h . k_p), exact
// int32.  The indexer heads form the M side (16 rows) of v_mfma_i32_16x16x64_i8 and 16 cached
// positions the N side, so one instruction scores 16 positions for 16 heads over 64 key bytes.
// Every key byte is read once with 16-byte loads; a wave covers 64 positions (one 8 KB page at
// the 64-token, 128-byte layout) per step.
//
// Selection (trnrt summary, "The interesting bit": the top 2,048 positions are kept; ties go to
// the lower position).  Radix select on the exact integer scores:
//   pass 1 (fused into scoring): a log-linear histogram (exact below 256, then 128 bins per
//            binade) locates the bin holding the k-th largest score;
//   refine:  4,096-bin histograms of the scores inside [lo, hi] narrow the range until lo == hi;
//   count:   per 4,096-position chunk, how many scores are > T and == T;
//   write:   an ordered compaction: a position is kept if its score is > T, or == T and fewer than
//            `need` equal scores precede it; its output slot is the number of kept positions
//            before it, so the list comes out in ascending position order.
// Each histogram is turned into the next range at the start of the following kernel, by every one of
// its workgroups (the same deterministic pick, from 16 KB that the kernel boundary made visible);
// workgroup 0 records the result for later kernels.  No workgroup waits on, or fences for, another:
// on this part an in-kernel device-scope fence writes back the whole L2 of the XCD, which costs far
// more than recomputing a 4,096-bin pick.
#include "dl_common.h"
#include "dl_internal.h"

namespace dl {

static constexpr int NB1 = 256 + 23 * 128;  // log-linear bins covering 0 .. 2^31-1
static constexpr int NB2 = 4096;
static constexpr int SCORE_POS_PER_BLOCK = 1024;  // 4 waves x 4 steps x 64 positions
static constexpr int SEL_CHUNK = 4096;            // 256 threads x 16 positions

// Rows and sequences: with R query rows per sequence (multi-row decode), row i belongs to sequence i / R and
// is the token at position seq_lens[i / R] - R + i % R, so it sees the positions before and including its own
// (causal among the R rows).  R = 1 is ordinary decode.
// With pool > 1 (pool-granular selection) the scored and selected items are pools of `pool` consecutive
// positions, keyed by a separate pool-key cache; a row's length is then counted in pools (the last may be
// partial).
__device__ __forceinline__ int row_len(const int32_t *seq_lens, int row, int R, int pool = 1)
{
    const int L = seq_lens[row / R] - (R - 1 - row % R);
    return L > 0 ? (L + pool - 1) / pool : 0;
}

__device__ __forceinline__ int bin1_of(int s)
{
    if (s < 256) return s;
    int n = 31 - __clz(s);  // 8 .. 30
    return 256 + (n - 8) * 128 + ((s >> (n - 7)) & 127);
}
__device__ __forceinline__ void bin1_range(int b, int &lo, int &hi)
{
    if (b < 256) { lo = hi = b; return; }
    int n = 8 + (b - 256) / 128, m = (b - 256) % 128;
    lo = (128 + m) << (n - 7);
    hi = lo + (1 << (n - 7)) - 1;
}

// Inclusive scan of one int across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Largest bin b with (count of bins >= b) >= k, and the count strictly above it.  Called by all 256
// threads of a workgroup: the histogram (finished by an earlier kernel) is copied into LDS with all loads
// in flight at once, the 256 segment sums are suffix-scanned, and the one thread whose segment holds the
// k-th largest score walks it.
template <int NBINS>
__device__ void block_pick(const unsigned *gh, unsigned *sh, int k, int *s_tmp, int &bin_out, int &above_out)
{
    constexpr int PER = (NBINS + 255) / 256;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    unsigned v[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int b = i * 256 + tid;
        v[i] = b < NBINS ? gh[b] : 0u;
    }
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int b = i * 256 + tid;
        if (b < NBINS) sh[b] = v[i];
    }
    __syncthreads();
    // thread tid owns segment t = 255 - tid (bins [t*PER, (t+1)*PER)), so a prefix scan over tid is a
    // suffix scan over the bins
    const int t = 255 - tid;
    int seg = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int b = t * PER + i;
        if (b < NBINS) seg += (int)sh[b];
    }
    int inc = wave_incl_scan(seg);
    if (lane == 63) s_tmp[wave] = inc;
    if (tid == 0) { s_tmp[256] = 0; s_tmp[257] = 0; }
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; w++) before += s_tmp[w];
    inc += before;
    const int exc = inc - seg;  // bins above my segment
    if (inc >= k && exc < k) {
        int cum = exc, bin = t * PER;
        for (int i = PER - 1; i >= 0; i--) {
            const int b = t * PER + i;
            if (b >= NBINS) continue;
            const int hcount = (int)sh[b];
            if (cum + hcount >= k) { bin = b; break; }
            cum += hcount;
        }
        s_tmp[256] = bin;
        s_tmp[257] = cum;
    }
    __syncthreads();
    bin_out = s_tmp[256];
    above_out = s_tmp[257];
    __syncthreads();
}

// The selection state after one more histogram: pass 1 uses the log-linear bins, later passes 4,096
// equal bins spanning the current [lo, hi].  A finished state passes through unchanged.
template <bool FIRST>
__device__ SelState advance(const SelState prev, const unsigned *gh, int top_k, unsigned *sh, int *s_tmp)
{
    if (prev.done) return prev;
    SelState s = prev;
    int bin, above;
    if (FIRST) {
        block_pick<NB1>(gh, sh, top_k, s_tmp, bin, above);
        int lo, hi;
        bin1_range(bin, lo, hi);
        s.lo = lo; s.hi = hi; s.above = above;
    } else {
        const unsigned lo = (unsigned)prev.lo, hi = (unsigned)prev.hi;
        const int shift = max(0, (32 - __clz(hi - lo)) - 12);
        block_pick<NB2>(gh, sh, top_k - prev.above, s_tmp, bin, above);
        const unsigned nlo = lo + ((unsigned)bin << shift);
        const unsigned nhi = min(hi, nlo + ((1u << shift) - 1u));
        s.lo = (int)nlo; s.hi = (int)nhi; s.above = prev.above + above;
    }
    if (s.lo == s.hi) { s.done = 1; s.need = top_k - s.above; }
    return s;
}

// Per-row initial selection state; clears the histograms of all passes.
__global__ void k_sel_init(const int32_t *seq_lens, int R, int pool, int B, int top_k, unsigned *hist1,
                           unsigned *hist2, SelState *st)
{
    const int b = blockIdx.x;
    for (int i = threadIdx.x; i < NB1; i += blockDim.x) hist1[(long)b * NB1 + i] = 0;
    for (int i = threadIdx.x; i < 2 * NB2; i += blockDim.x) hist2[(long)b * 2 * NB2 + i] = 0;
    if (threadIdx.x == 0) {
        int L = row_len(seq_lens, b, R, pool);
        SelState s;
        s.n_sel = min(L, top_k);
        if (L <= top_k) {  // keep everything: every score (>= 0) is above T = -1
            s.lo = s.hi = -1; s.above = L; s.done = 1; s.need = 0;
        } else {
            s.lo = 0; s.hi = 0x7FFFFFFF; s.above = 0; s.done = 0; s.need = 0;
        }
        s.pad0 = s.pad1 = 0;
        st[b] = s;  // state 0 of row b
    }
}

// Scores of 1,024 positions of one sequence per workgroup.  NHG groups of 16 indexer heads, KCH chunks of 64 key
// bytes, RW query rows per sequence: every key is loaded once and scored against all RW rows (RW x NHG matrix
// instructions per 16 positions and 64 key bytes), each row keeping the positions it sees.
template <int NHG, int KCH, int RW>
__global__ __launch_bounds__(256) void k_index_score(const int8_t *__restrict__ q_idx, const int8_t *__restrict__ k_pool,
                                                     const int32_t *__restrict__ page_table,
                                                     const int32_t *__restrict__ seq_lens, int pool, int max_pages,
                                                     int ps_shift, int HI, int DI, int32_t *__restrict__ scores,
                                                     long Lmax, unsigned *__restrict__ hist1)
{
    __shared__ unsigned s_hist[RW][NB1];
    const int sq = blockIdx.y;
    // items (positions, or pools of `pool` positions) of the sequence; row r sees the items of its first
    // seq_lens - (RW - 1 - r) positions
    const int L = row_len(seq_lens, sq * RW + RW - 1, RW, pool);
    const long blk0 = (long)blockIdx.x * SCORE_POS_PER_BLOCK;
    if (blk0 >= L) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, lg = lane >> 4;
    for (int i = tid; i < RW * NB1; i += 256) (&s_hist[0][0])[i] = 0;

    // A operand: q rows (indexer heads) for this lane: head hg*16+ln, bytes kc*64 + lg*16 .. +16
    v4i A[RW][NHG][KCH];
#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
        for (int hg = 0; hg < NHG; hg++)
#pragma unroll
            for (int kc = 0; kc < KCH; kc++) {
                int h = hg * 16 + ln, d = kc * 64 + lg * 16;
                A[r][hg][kc] = (h < HI && d < DI) ? ldg16(q_idx + (((long)sq * RW + r) * HI + h) * DI + d)
                                                  : v4i{0, 0, 0, 0};
            }
    const int32_t *pt = page_table + (long)sq * max_pages;
    const int ps_mask = (1 << ps_shift) - 1;
    // cache rows of every position this lane loads (step st, group sg: position g0(st) + sg*16 + ln), all
    // page-table reads in flight at once
    long row[4][4];
#pragma unroll
    for (int st = 0; st < 4; st++)
#pragma unroll
        for (int sg = 0; sg < 4; sg++) {
            const long pos = blk0 + (long)(st * 4 + wave) * 64 + sg * 16 + ln;
            row[st][sg] = pos < L ? ((long)pt[pos >> ps_shift] << ps_shift) + (pos & ps_mask) : -1;
        }
    __syncthreads();
    // keys of step st: 4 groups of 16 positions x KCH chunks of 64 bytes; two steps in flight
    auto load_keys = [&](int st, v4i (&Bk)[4][KCH]) {
#pragma unroll
        for (int sg = 0; sg < 4; sg++)
#pragma unroll
            for (int kc = 0; kc < KCH; kc++) {
                const int d = kc * 64 + lg * 16;
                // streaming loads: every key byte is read once per step
                Bk[sg][kc] = (row[st][sg] >= 0 && d < DI)
                                 ? __builtin_nontemporal_load((const v4i *)(k_pool + row[st][sg] * DI + d))
                                 : v4i{0, 0, 0, 0};
            }
    };
    v4i K0[4][KCH], K1[4][KCH];
    load_keys(0, K0);
    load_keys(1, K1);
#pragma unroll
    for (int st = 0; st < 4; st++) {
        const long g0 = blk0 + (long)(st * 4 + wave) * 64;  // this wave's 64 positions
        v4i (&Bk)[4][KCH] = (st & 1) ? K1 : K0;
        int mine[RW];
#pragma unroll
        for (int r = 0; r < RW; r++) mine[r] = 0;
#pragma unroll
        for (int sg = 0; sg < 4; sg++) {
#pragma unroll
            for (int r = 0; r < RW; r++) {
                int part = 0;
#pragma unroll
                for (int hg = 0; hg < NHG; hg++) {
                    v4i acc = {0, 0, 0, 0};
#pragma unroll
                    for (int kc = 0; kc < KCH; kc++)
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[r][hg][kc], Bk[sg][kc], acc, 0, 0, 0);
                    // lane holds heads hg*16 + 4*lg + i of position sg*16 + ln
                    part += max(acc[0], 0) + max(acc[1], 0) + max(acc[2], 0) + max(acc[3], 0);
                }
                part += __shfl_xor(part, 16, 64);
                part += __shfl_xor(part, 32, 64);
                if (lg == sg) mine[r] = part;
            }
        }
        if (st + 2 < 4) load_keys(st + 2, Bk);  // this buffer is free again
        const long pos = g0 + lane;
#pragma unroll
        for (int r = 0; r < RW; r++) {
            if (pos < row_len(seq_lens, sq * RW + r, RW, pool)) {
                scores[((long)sq * RW + r) * Lmax + pos] = mine[r];
                atomicAdd(&s_hist[r][bin1_of(mine[r])], 1u);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RW; r++) {
        unsigned *gh = hist1 + ((long)sq * RW + r) * NB1;
        for (int i = tid; i < NB1; i += 256) {
            const unsigned v = s_hist[r][i];
            if (v) atomicAdd(gh + i, v);
        }
    }
}

__device__ __forceinline__ void load16(const int32_t *sc, long p0, int L, int v[16])
{
    if (p0 + 16 <= L) {
        const v4i *q = (const v4i *)(sc + p0);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v4i t = q[i];
            v[4 * i] = t[0]; v[4 * i + 1] = t[1]; v[4 * i + 2] = t[2]; v[4 * i + 3] = t[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = (p0 + i < L) ? sc[p0 + i] : INT32_MIN;
    }
}

// One refinement pass (PASS = 1, 2): advance the state with histogram PASS, then histogram the scores
// inside the new [lo, hi] with 4,096 bins into histogram PASS + 1.
template <int PASS>
__global__ __launch_bounds__(256) void k_sel_refine(const int32_t *__restrict__ scores, long Lmax,
                                                    const int32_t *__restrict__ seq_lens, int R, int pool, int top_k,
                                                    const unsigned *__restrict__ hist_in, unsigned *__restrict__ hist_out,
                                                    SelState *__restrict__ st, int B)
{
    __shared__ unsigned s_hist[NB2 > NB1 ? NB2 : NB1];
    __shared__ int s_tmp[260];
    const int b = blockIdx.y;
    const int L = row_len(seq_lens, b, R, pool);
    const long c0 = (long)blockIdx.x * SEL_CHUNK;
    if (c0 >= L && blockIdx.x != 0) return;
    const int tid = threadIdx.x;
    const SelState prev = st[(long)(PASS - 1) * B + b];
    const SelState cur = PASS == 1 ? advance<true>(prev, hist_in + (long)b * NB1, top_k, s_hist, s_tmp)
                                   : advance<false>(prev, hist_in + (long)b * NB2, top_k, s_hist, s_tmp);
    if (blockIdx.x == 0 && tid == 0) st[(long)PASS * B + b] = cur;
    if (c0 >= L || cur.done) return;
    const unsigned lo = (unsigned)cur.lo, hi = (unsigned)cur.hi;
    const int shift = max(0, (32 - __clz(hi - lo)) - 12);
    __syncthreads();
    for (int i = tid; i < NB2; i += 256) s_hist[i] = 0;
    __syncthreads();
    // the thread's 16 consecutive scores, all loads in flight at once (positions past L read INT32_MIN,
    // which is outside every range)
    int v[16];
    load16(scores + (long)b * Lmax, c0 + (long)tid * 16, L, v);
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const unsigned x = (unsigned)v[i];
        if (v[i] >= 0 && x >= lo && x <= hi) atomicAdd(&s_hist[(x - lo) >> shift], 1u);
    }
    __syncthreads();
    unsigned *gh = hist_out + (long)b * NB2;
    for (int i = tid; i < NB2; i += 256) {
        const unsigned v = s_hist[i];
        if (v) atomicAdd(gh + i, v);
    }
}

// Per chunk: how many scores are > T and == T.
__global__ __launch_bounds__(256) void k_sel_count(const int32_t *__restrict__ scores, long Lmax,
                                                   const int32_t *__restrict__ seq_lens, int R, int pool, int top_k,
                                                   const unsigned *__restrict__ hist3, SelState *__restrict__ st, int B,
                                                   int nchunk, int *__restrict__ cnt)
{
    __shared__ unsigned s_hist[NB2];
    __shared__ int s_tmp[260];
    __shared__ int s_red[2][4];
    const int b = blockIdx.y;
    const int L = row_len(seq_lens, b, R, pool);
    const long c0 = (long)blockIdx.x * SEL_CHUNK;
    if (c0 >= L && blockIdx.x != 0) return;
    const int tid = threadIdx.x;
    const SelState cur = advance<false>(st[2L * B + b], hist3 + (long)b * NB2, top_k, s_hist, s_tmp);
    if (blockIdx.x == 0 && tid == 0) st[3L * B + b] = cur;
    if (c0 >= L) return;
    const int T = cur.lo;
    int v[16];
    load16(scores + (long)b * Lmax, c0 + (long)tid * 16, L, v);
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        gt += v[i] > T;
        eq += v[i] == T;
    }
    gt = wave_sum_i(gt);
    eq = wave_sum_i(eq);
    if ((tid & 63) == 0) { s_red[0][tid >> 6] = gt; s_red[1][tid >> 6] = eq; }
    __syncthreads();
    if (tid == 0) {
        long o = ((long)b * nchunk + blockIdx.x) * 2;
        cnt[o] = s_red[0][0] + s_red[0][1] + s_red[0][2] + s_red[0][3];
        cnt[o + 1] = s_red[1][0] + s_red[1][1] + s_red[1][2] + s_red[1][3];
    }
}

// Ordered compaction of the kept positions of one chunk.
__global__ __launch_bounds__(256) void k_sel_write(const int32_t *__restrict__ scores, long Lmax,
                                                   const int32_t *__restrict__ seq_lens, int R, int pool, const SelState *__restrict__ st,
                                                   int nchunk, const int *__restrict__ cnt, int top_k,
                                                   int32_t *__restrict__ sel, int32_t *__restrict__ sel_score)
{
    __shared__ int s_w[2][4];
    __shared__ int s_base[2];
    const int b = blockIdx.y;
    const int L = row_len(seq_lens, b, R, pool);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const SelState s = st[3L * gridDim.y + b];
    // pool > 1: slot k holds positions [k pool, (k + 1) pool) of the output row (the kept pool's positions,
    // those at or past the row's last position written as -1); sel_score holds one score per slot
    int32_t *so = sel + (long)b * top_k * pool;
    int32_t *ss = sel_score ? sel_score + (long)b * top_k : nullptr;
    const int plen = pool > 1 ? row_len(seq_lens, b, R) : 0;  // positions the row sees
    if (blockIdx.x == 0) {  // padding of the unused slots
        for (int i = s.n_sel * pool + tid; i < top_k * pool; i += 256) so[i] = -1;
        if (ss)
            for (int i = s.n_sel + tid; i < top_k; i += 256) ss[i] = 0;
    }
    // pools of 4 or more positions go out as 16-byte stores when the output is 16-byte aligned
    const bool vec = pool >= 4 && ((uintptr_t)sel & 15) == 0;
    auto put = [&](int slot, int item, int score) {
        if (pool == 1) {
            so[slot] = item;
        } else if (vec) {
            for (int j = 0; j < pool; j += 4) {
                const int p = item * pool + j;
                *(v4i *)(so + slot * pool + j) =
                    v4i{p < plen ? p : -1, p + 1 < plen ? p + 1 : -1, p + 2 < plen ? p + 2 : -1, p + 3 < plen ? p + 3 : -1};
            }
        } else {
            for (int j = 0; j < pool; j++) {
                const int p = item * pool + j;
                so[slot * pool + j] = p < plen ? p : -1;
            }
        }
        if (ss) ss[slot] = score;
    };
    const long c0 = (long)blockIdx.x * SEL_CHUNK;
    if (c0 >= L) return;
    const int T = s.lo, need = s.need;
    // counts of all earlier chunks of this row
    int pg = 0, pe = 0;
    for (int c = tid; c < (int)blockIdx.x; c += 256) {
        pg += cnt[((long)b * nchunk + c) * 2];
        pe += cnt[((long)b * nchunk + c) * 2 + 1];
    }
    pg = wave_sum_i(pg);
    pe = wave_sum_i(pe);
    if (lane == 0) { s_w[0][wave] = pg; s_w[1][wave] = pe; }
    __syncthreads();
    if (tid == 0) {
        s_base[0] = s_w[0][0] + s_w[0][1] + s_w[0][2] + s_w[0][3];
        s_base[1] = s_w[1][0] + s_w[1][1] + s_w[1][2] + s_w[1][3];
    }
    __syncthreads();
    const int base_g = s_base[0], base_e = s_base[1];
    const long p0 = c0 + (long)tid * 16;
    int v[16];
    load16(scores + (long)b * Lmax, p0, L, v);
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        gt += v[i] > T;
        eq += v[i] == T;
    }
    // exclusive scan of (gt, eq) over the 256 threads
    int ig = wave_incl_scan(gt), ie = wave_incl_scan(eq);
    __syncthreads();
    if (lane == 63) { s_w[0][wave] = ig; s_w[1][wave] = ie; }
    __syncthreads();
    int wg = 0, we = 0;
    for (int w = 0; w < wave; w++) { wg += s_w[0][w]; we += s_w[1][w]; }
    int g = base_g + wg + ig - gt;  // kept-above scores before my first position
    int e = base_e + we + ie - eq;  // equal scores before my first position
#pragma unroll
    for (int i = 0; i < 16; i++) {
        int sv = v[i];
        // slots outside [0, top_k) are dropped: only an inconsistent state (never produced from consistent
        // counts) can ask for them, and they would lie outside the row
        if (sv > T) {
            int slot = g + min(e, need);
            if (slot >= 0 && slot < top_k) put(slot, (int)(p0 + i), sv);
            g++;
        } else if (sv == T) {
            if (e < need) {
                int slot = g + e;
                if (slot >= 0 && slot < top_k) put(slot, (int)(p0 + i), sv);
            }
            e++;
        }
    }
}

// ------------------------------------------------------------------ host side
static int max_len(const dl_pages &pg) { return pg.max_pages_per_seq * pg.page_size; }

void topk_ws_layout(Ws &w, const dl_pages &pg, TopkWs &t, int R, int pool)
{
    const long B = (long)pg.batch * R, Lmax = max_len(pg) / pool;  // one selection per row, over items
    const long nchunk = (Lmax + SEL_CHUNK - 1) / SEL_CHUNK;
    t.scores = w.take<int32_t>(B * Lmax);
    t.hist1 = w.take<unsigned>(B * NB1);
    t.hist2 = w.take<unsigned>(B * 2 * NB2);  // histograms of passes 2 and 3
    t.state = w.take<SelState>(4 * B);        // state after 0 .. 3 histograms
    t.cnt = w.take<int>(B * nchunk * 2);
}

template <int NHG, int KCH>
static void launch_score(dim3 g, hipStream_t s, const int8_t *q, const int8_t *kp, const dl_pages &pg, int ps_shift,
                         int HI, int DI, const TopkWs &t, long Lmax, int R, int pool)
{
#define DL_SCORE_R(R_)                                                                                              \
    if (R == R_)                                                                                                    \
        hipLaunchKernelGGL((k_index_score<NHG, KCH, R_>), g, dim3(256), 0, s, q, kp, pg.page_table, pg.seq_lens,   \
                           pool, pg.max_pages_per_seq, ps_shift, HI, DI, t.scores, Lmax, t.hist1);
    DL_SCORE_R(1) DL_SCORE_R(2) DL_SCORE_R(3) DL_SCORE_R(4)
#undef DL_SCORE_R
}

int launch_indexer_topk(const dl_pages &pg, const int8_t *q_idx, const int8_t *k_pool, int HI, int DI, int top_k,
                        int32_t *sel, int32_t *sel_score, const TopkWs &t, hipStream_t s, int R, int pool)
{
    if (R < 1 || R > DL_MAX_ROWS_PER_SEQ) return fail(DL_ERR_UNSUPPORTED, "rows per sequence %d (1..%d)", R, DL_MAX_ROWS_PER_SEQ);
    if (pool < 1 || pool > pg.page_size || (pool & (pool - 1))) return fail(DL_ERR_UNSUPPORTED, "pool %d", pool);
    const int B = pg.batch * R;  // rows
    const long Lmax = max_len(pg) / pool;  // items per row
    // the key cache holds page_size / pool items per page
    const int ps_shift = __builtin_ctz((unsigned)(pg.page_size / pool));
    const int nchunk = (int)((Lmax + SEL_CHUNK - 1) / SEL_CHUNK);
    hipLaunchKernelGGL(k_sel_init, dim3(B), dim3(256), 0, s, pg.seq_lens, R, pool, B, top_k, t.hist1, t.hist2,
                       t.state);
    dim3 gs((unsigned)((Lmax + SCORE_POS_PER_BLOCK - 1) / SCORE_POS_PER_BLOCK), pg.batch);
    const int nhg = (HI + 15) / 16, kch = (DI + 63) / 64;
#define DL_SCORE_CASE(H_, K_) \
    if (nhg == H_ && kch == K_) launch_score<H_, K_>(gs, s, q_idx, k_pool, pg, ps_shift, HI, DI, t, Lmax, R, pool); else
    DL_SCORE_CASE(1, 1) DL_SCORE_CASE(1, 2) DL_SCORE_CASE(1, 3) DL_SCORE_CASE(1, 4)
    DL_SCORE_CASE(2, 1) DL_SCORE_CASE(2, 2) DL_SCORE_CASE(2, 3) DL_SCORE_CASE(2, 4)
    DL_SCORE_CASE(3, 1) DL_SCORE_CASE(3, 2) DL_SCORE_CASE(3, 3) DL_SCORE_CASE(3, 4)
    DL_SCORE_CASE(4, 1) DL_SCORE_CASE(4, 2) DL_SCORE_CASE(4, 3) DL_SCORE_CASE(4, 4)
    return fail(DL_ERR_UNSUPPORTED, "indexer shape heads=%d dim=%d", HI, DI);
#undef DL_SCORE_CASE
    dim3 gc(nchunk, B);
    // 31-bit scores: pass 1 leaves a range of at most 2^23 values; each refinement takes 12 bits, so the
    // state after histogram 3 is always final.
    unsigned *h2 = t.hist2, *h3 = t.hist2 + (long)B * NB2;
    hipLaunchKernelGGL((k_sel_refine<1>), gc, dim3(256), 0, s, t.scores, Lmax, pg.seq_lens, R, pool, top_k, t.hist1,
                       h2, t.state, B);
    hipLaunchKernelGGL((k_sel_refine<2>), gc, dim3(256), 0, s, t.scores, Lmax, pg.seq_lens, R, pool, top_k, h2, h3,
                       t.state, B);
    hipLaunchKernelGGL(k_sel_count, gc, dim3(256), 0, s, t.scores, Lmax, pg.seq_lens, R, pool, top_k, h3, t.state, B,
                       nchunk, t.cnt);
    hipLaunchKernelGGL(k_sel_write, gc, dim3(256), 0, s, t.scores, Lmax, pg.seq_lens, R, pool, t.state, nchunk,
                       t.cnt, top_k, sel, sel_score);
    return hip_check("indexer_topk");
}

}  // namespace dl
