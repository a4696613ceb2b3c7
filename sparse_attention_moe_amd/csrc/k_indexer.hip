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
// the lower position), exact on the integer scores:
//   histogram (fused into scoring): a log-linear histogram (exact below 256, then 128 bins per
//            binade) locates the bin [lo, hi] holding the k-th largest score and the count above it;
//   mark:    one pass over the scores: positions scoring above hi are set in a per-row bitmap (each
//            word written whole by the workgroup owning its positions), positions inside [lo, hi]
//            go with their scores to the workgroup's own region of the candidate list, with a count;
//   final:   one workgroup per row keeps the `need` best candidates by a radix select on a unique key
//            (score above, complemented position below, so ties go to the lower position), sets their
//            bits, then compacts the bitmap in position order, so the list comes out ascending.
// Every mark workgroup picks the bin from the histogram (the same deterministic pick, made visible by
// the kernel boundary); workgroup 0 records it for the final kernel.  No device-wide barrier: on this part one
// costs far more than a kernel boundary.  The one wait inside a kernel is the scoring workgroups' wait for their
// sequence's first workgroup to have cleared the histograms (a per-launch stamp, read once at their end).
#include "dl_common.h"
#include "dl_internal.h"

#include <algorithm>
#include <atomic>
#include <chrono>
#include <stdint.h>
#include <unistd.h>

namespace dl {

static constexpr int NB1 = 256 + 23 * 128;  // log-linear bins covering 0 .. 2^31-1
// Scoring workgroups of score_wpb() waves, 4 steps of 64 positions each.  Sixteen waves fill a compute unit with
// one workgroup, so its barrier after the page lookups holds back every key load on the unit until all of the
// unit's lookups are back: with four workgroups per unit, the lookups of the later ones queued behind the key
// stream of the earlier ones (measured: back at 3 us for the first two, 17 us for the last).  Shapes whose
// registers do not fit four waves per SIMD (128 each) keep workgroups of four waves.
__host__ __device__ constexpr int score_wpb(int NHG, int KCH, int RW)
{
    return (KCH == 1 && NHG * RW <= 9) || (KCH == 2 && NHG * RW <= 2) ? 16 : 4;
}
static constexpr int SEL_CHUNK = 4096;  // select passes: 256 threads x 16 items

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

// Where the selection threshold lies, from the row's log-linear histogram: items scoring above hi are kept,
// `need` of the items inside [lo, hi] are kept.  A row of at most top_k items keeps everything (hi = -1: every
// score is >= 0).  Called by all 256 threads of a workgroup.
__device__ Thr threshold(const unsigned *gh, int L, int top_k, unsigned *sh, int *s_tmp)
{
    Thr t;
    if (L <= top_k) {
        t.lo = 0x7FFFFFFF; t.hi = -1; t.need = 0;
        return t;
    }
    int bin, above;
    block_pick<NB1>(gh, sh, top_k, s_tmp, bin, above);
    bin1_range(bin, t.lo, t.hi);
    t.need = top_k - above;
    return t;
}

// Scores of score_wpb() x 256 positions of one sequence per workgroup.  NHG groups of 16 indexer heads, KCH
// chunks of 64 key bytes, RW query rows per sequence: every key is loaded once and scored against all RW rows (RW x
// NHG matrix instructions per 16 positions and 64 key bytes), each row keeping the positions it sees.
template <int NHG, int KCH, int RW>
__global__ __launch_bounds__(score_wpb(NHG, KCH, RW) * 64) void k_index_score(const int8_t *__restrict__ q_idx, const int8_t *__restrict__ k_pool,
                                                     const int32_t *__restrict__ page_table,
                                                     const int32_t *__restrict__ seq_lens, int pool, int max_pages,
                                                     int ps_shift, int HI, int DI, int32_t *__restrict__ scores,
                                                     long Lmax, unsigned *__restrict__ hist1,
                                                     unsigned long long *__restrict__ hflag, unsigned long long epoch,
                                                     int tiles)
{
    constexpr int SCORE_WPB = score_wpb(NHG, KCH, RW);
    constexpr int SCORE_POS_PER_BLOCK = SCORE_WPB * 4 * 64;
    __shared__ unsigned s_hist[RW][NB1];
    const int sq = blockIdx.y;
    const long blk0 = (long)blockIdx.x * SCORE_POS_PER_BLOCK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, lg = lane >> 4;
    // The sequence's first workgroup clears its rows' histograms and then stamps the sequence's flag with this
    // launch's epoch (a value no earlier launch used); every workgroup adds to the histograms only once it has
    // read that stamp.  The clear's stores write through to memory and are complete before the stamp is
    // written, and the histogram atomics are device-scope, so they land on the cleared words.  The first
    // workgroup of a sequence precedes the others in dispatch order, so it is resident or done when they wait.
    if (blockIdx.x == 0) {
        unsigned *gh = hist1 + (long)sq * RW * NB1;
        for (int i = tid; i < RW * NB1; i += SCORE_WPB * 64) st_dev(gh + i, 0u);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) st_dev(hflag + sq, epoch);
    }
    // The sequence's length, the query rows and the page-table entries of every position this lane loads are
    // read together, before the length is known (one round trip instead of two): the entries of positions
    // clamped to the page table's reach, and every read unconditional (a read under a condition is waited for on
    // its own), masked afterwards.  Positions past the end then take the workgroup's first position's row, and
    // their scores are never stored.
    const int32_t *pt = page_table + (long)sq * max_pages;
    const int ps_mask = (1 << ps_shift) - 1;
    const long pmax = ((long)max_pages << ps_shift) - 1;  // the last item the page table reaches
    int pe[4][4];
#pragma unroll
    for (int st = 0; st < 4; st++)
#pragma unroll
        for (int sg = 0; sg < 4; sg++) {
            const long pos = blk0 + (long)(st * SCORE_WPB + wave) * 64 + sg * 16 + ln;
            pe[st][sg] = pt[min(pos, pmax) >> ps_shift];
        }
    const int pe0 = pt[min(blk0, pmax) >> ps_shift];
    // A operand: q rows (indexer heads) for this lane: head hg*16+ln, bytes kc*64 + lg*16 .. +16 (zero past the
    // heads or the key dimension)
    v4i A[RW][NHG][KCH];
#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
        for (int hg = 0; hg < NHG; hg++)
#pragma unroll
            for (int kc = 0; kc < KCH; kc++) {
                const int h = min(hg * 16 + ln, HI - 1), d = min(kc * 64 + lg * 16, DI - 16);
                A[r][hg][kc] = ldg16(q_idx + (((long)sq * RW + r) * HI + h) * DI + d);
            }
#pragma unroll
    for (int hg = 0; hg < NHG; hg++)
#pragma unroll
        for (int kc = 0; kc < KCH; kc++)
            if (!(hg * 16 + ln < HI && kc * 64 + lg * 16 < DI))
#pragma unroll
                for (int r = 0; r < RW; r++) A[r][hg][kc] = v4i{0, 0, 0, 0};
    // items (positions, or pools of `pool` positions) of the sequence; row r sees the items of its first
    // seq_lens - (RW - 1 - r) positions
    const int L = row_len(seq_lens, sq * RW + RW - 1, RW, pool);
    if (blk0 >= L) return;
    for (int i = tid; i < RW * NB1; i += SCORE_WPB * 64) (&s_hist[0][0])[i] = 0;
    long row[4][4];
#pragma unroll
    for (int st = 0; st < 4; st++)
#pragma unroll
        for (int sg = 0; sg < 4; sg++) {
            const long pos = blk0 + (long)(st * SCORE_WPB + wave) * 64 + sg * 16 + ln;
            row[st][sg] = pos < L ? ((long)pe[st][sg] << ps_shift) + (pos & ps_mask)
                                  : ((long)pe0 << ps_shift) + (blk0 & ps_mask);
        }
    __syncthreads();
    // keys of step st: 4 groups of 16 positions x KCH chunks of 64 bytes; two steps in flight.  Key bytes past DI
    // (a last chunk narrower than 64) are read from inside the item (row-major) or its group (tiled) instead and
    // meet zero query columns, so they add nothing
    auto load_keys = [&](int st, v4i (&Bk)[4][KCH]) {
#pragma unroll
        for (int sg = 0; sg < 4; sg++)
#pragma unroll
            for (int kc = 0; kc < KCH; kc++) {
                const int d = min(kc * 64 + lg * 16, DI - 16);
                // streaming loads: every key byte is read once per step.  Tiled keys: the 64 lanes read the
                // item group's 1 KB chunk kc contiguously (lane = lg * 16 + ln, item ln of the group)
                const long off = tiles ? (row[st][sg] & ~15L) * DI + min(kc * 1024 + lane * 16, 16 * DI - 16)
                                       : row[st][sg] * DI + d;
                Bk[sg][kc] = __builtin_nontemporal_load((const v4i *)(k_pool + off));
            }
    };
    v4i K0[4][KCH], K1[4][KCH];
    load_keys(0, K0);
    load_keys(1, K1);
#pragma unroll
    for (int st = 0; st < 4; st++) {
        const long g0 = blk0 + (long)(st * SCORE_WPB + wave) * 64;  // this wave's 64 positions
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
    // the histograms are cleared once the sequence's flag holds this launch's epoch (read by one thread; the
    // barrier passes it on).  A bounded wait: the first workgroup stamps the flag within a few microseconds
    if (tid == 0) {
        unsigned long long f = ld_dev(hflag + sq);
        for (int it = 0; f != epoch && it < (1 << 22); it++) {
            __builtin_amdgcn_s_sleep(4);
            f = ld_dev(hflag + sq);
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RW; r++) {
        unsigned *gh = hist1 + ((long)sq * RW + r) * NB1;
        for (int i = tid; i < NB1; i += SCORE_WPB * 64) {
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

// Mark: per 4,096-item chunk of a row longer than top_k, the bitmap words of its items (bit set: score above
// the threshold bin), and its items inside the bin, with their scores, in the chunk's own region of the
// candidate list ([row][chunk * 4,096 + i]) with their count; workgroup 0 records the bin.
__global__ __launch_bounds__(256) void k_sel_mark(const int32_t *__restrict__ scores, long Lmax,
                                                  const int32_t *__restrict__ seq_lens, int R, int pool, int top_k,
                                                  const unsigned *__restrict__ hist1, unsigned *__restrict__ bits,
                                                  long Lw, int2 *__restrict__ cand, int32_t *__restrict__ ccnt,
                                                  int32_t *__restrict__ acnt, int nchunk, Thr *__restrict__ thr)
{
    __shared__ unsigned s_hist[NB1];
    __shared__ int s_tmp[260];
    __shared__ int s_w[4];
    __shared__ int s_a[4];
    const int b = blockIdx.y;
    const int L = row_len(seq_lens, b, R, pool);
    const long c0 = (long)blockIdx.x * SEL_CHUNK;
    if (L <= top_k || c0 >= L) return;  // short rows keep everything without a bitmap
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the thread's 16 consecutive scores, loaded while the bin is picked (items past L read INT32_MIN:
    // neither above hi nor inside the bin)
    int v[16];
    load16(scores + (long)b * Lmax, c0 + (long)tid * 16, L, v);
    const Thr t = threshold(hist1 + (long)b * NB1, L, top_k, s_hist, s_tmp);
    if (blockIdx.x == 0 && tid == 0) thr[b] = t;
    unsigned m = 0;
    int nc = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        if (v[i] > t.hi) m |= 1u << i;
        else if (v[i] >= t.lo) nc++;
    }
    // two threads fill one 32-bit word: the even one the low half
    const unsigned mo = (unsigned)__shfl_xor((int)m, 1, 64);
    if ((tid & 1) == 0) bits[(long)b * Lw + (c0 >> 5) + (tid >> 1)] = m | (mo << 16);
    // candidates: exclusive scan over the workgroup into the chunk's region; and the chunk's marked items
    const int inc = wave_incl_scan(nc);
    const int na = wave_sum_i(__popc(m));
    if (lane == 63) s_w[wave] = inc;
    if (lane == 0) s_a[wave] = na;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; w++) before += s_w[w];
    if (tid == 0) {
        ccnt[(long)b * nchunk + blockIdx.x] = s_w[0] + s_w[1] + s_w[2] + s_w[3];
        acnt[(long)b * nchunk + blockIdx.x] = s_a[0] + s_a[1] + s_a[2] + s_a[3];
    }
    int o = before + inc - nc;
    int2 *cr = cand + (long)b * nchunk * SEL_CHUNK + c0;
#pragma unroll
    for (int i = 0; i < 16; i++)
        if (v[i] <= t.hi && v[i] >= t.lo) cr[o++] = int2{(int)(c0 + (long)tid * 16 + i), v[i]};
}

static constexpr int FCAP = 4096;   // candidates whose keys the final kernel holds in LDS; more are re-read
static constexpr int FCH = 2048;    // chunks per row the final kernel handles (rows of up to 8M items)
static constexpr int FCPW = 2;      // chunks a final workgroup compacts (256 bitmap words: one per thread)
static constexpr int FBW = FCPW * (SEL_CHUNK / 32);

// Final: gridDim.x workgroups per row, workgroup g owning chunks [FCPW g, FCPW (g + 1)).  Rows of at most top_k
// items keep items 0 .. L-1.  In longer rows every workgroup finds the same `need` best candidates (the row has
// few: the items of one histogram bin): with at most 256 in LDS, each candidate's rank among them; otherwise a
// radix select, most significant 8-bit digit first, of the need-th largest key ((score - lo) << PB |
// (2^PB - 1 - item)); keys are unique, so exactly `need` keys match the final prefix or exceed it.  The kept
// items before its chunks (the marked counts of the earlier chunks and their kept candidates) give the
// workgroup's first output slot; it then adds its kept candidates' bits to its bitmap words and compacts them
// in item order, so the list comes out ascending and every slot is written by exactly one workgroup.
// pool > 1: slot k holds items' positions [k pool, (k + 1) pool), those at or past the row's length as -1.
__global__ __launch_bounds__(256) void k_sel_final(const int32_t *__restrict__ scores, long Lmax,
                                                   const int32_t *__restrict__ seq_lens, int R, int pool, int top_k,
                                                   const unsigned *__restrict__ bits, long Lw,
                                                   const int2 *__restrict__ cand, const int32_t *__restrict__ ccnt,
                                                   const int32_t *__restrict__ acnt, int nchunk,
                                                   const Thr *__restrict__ thr, int PB, int32_t *__restrict__ sel,
                                                   int32_t *__restrict__ sel_score)
{
    typedef unsigned long long u64;
    __shared__ unsigned s_hist[256];
    __shared__ int s_off[FCH + 1];
    __shared__ int s_kc[FCH];       // kept candidates per chunk (chunks before and in this workgroup's range)
    // the candidates' keys, then (once the kept ones are known) this workgroup's kept items in order
    __shared__ union {
        u64 key[FCAP];
        int out[FBW * 32];
    } s_ko;
    static_assert(FBW * 32 * sizeof(int) <= FCAP * sizeof(u64), "kept items fit the keys' LDS");
    u64 *s_key = s_ko.key;
    int *s_out = s_ko.out;
    __shared__ unsigned s_bm[FBW];  // bits of the kept candidates in this workgroup's words
    __shared__ int s_w[4];
    __shared__ int s_pick[3];
    const int b = blockIdx.y, g = blockIdx.x;
    const int L = row_len(seq_lens, b, R, pool);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t *sr = scores + (long)b * Lmax;
    int32_t *so = sel + (long)b * top_k * pool;
    int32_t *ss = sel_score ? sel_score + (long)b * top_k : nullptr;
    const int plen = pool > 1 ? row_len(seq_lens, b, R) : 0;  // positions the row sees
    const int n_sel = min(L, top_k);
    if (g == 0) {  // padding of the unused slots
        for (int i = n_sel * pool + tid; i < top_k * pool; i += 256) so[i] = -1;
        if (ss)
            for (int i = n_sel + tid; i < top_k; i += 256) ss[i] = 0;
    }
    // pools of 4 or more positions go out as 16-byte stores when the output is 16-byte aligned
    const bool vec = pool >= 4 && ((uintptr_t)sel & 15) == 0;
    auto put = [&](int slot, int item) {
        if (slot < 0 || slot >= top_k) return;  // only an inconsistent list could ask; it would leave the row
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
        if (ss) ss[slot] = sr[item];
    };
    const int i0 = g * FCPW * SEL_CHUNK;  // this workgroup's first item
    if (L <= top_k) {
        for (int i = i0 + tid; i < min(L, i0 + FCPW * SEL_CHUNK); i += 256) put(i, i);
        return;
    }
    const int nch = (L + SEL_CHUNK - 1) / SEL_CHUNK;
    const int ca = g * FCPW, cb = min(nch, ca + FCPW);  // this workgroup's chunks
    if (ca >= nch) return;
    const unsigned *br = bits + (long)b * Lw;
    const int2 *cr = cand + (long)b * nchunk * SEL_CHUNK;
    const Thr t = thr[b];
    // this thread's bitmap word and the first round of the two count loops below, loaded first and together
    // (unconditional, with clamped indices: a load under a condition is waited for on its own)
    const int nw = (L + 31) >> 5;
    const int wi = ca * (SEL_CHUNK / 32) + tid;
    const unsigned wv = br[min(wi, nw - 1)];
    const int a0 = acnt[(long)b * nchunk + min(tid, max(ca - 1, 0))];
    const int n0 = ccnt[(long)b * nchunk + min(tid, nch - 1)];
    unsigned word = wi < nw && tid < (cb - ca) * (SEL_CHUNK / 32) ? wv : 0u;
    // marked items of the chunks before this workgroup's
    int abefore = 0;
    for (int c0 = 0; c0 < ca; c0 += 256) {
        const int ch = c0 + tid;
        const int v = c0 == 0 ? a0 : acnt[(long)b * nchunk + min(ch, ca - 1)];
        abefore += wave_sum_i(ch < ca ? v : 0);
    }
    if (lane == 0) s_w[wave] = abefore;
    __syncthreads();
    abefore = s_w[0] + s_w[1] + s_w[2] + s_w[3];
    __syncthreads();
    // candidate counts of the row's chunks -> offsets of each chunk's run in the candidate order
    {
        int carry = 0;
        for (int c0 = 0; c0 < nch; c0 += 256) {
            const int ch = c0 + tid;
            const int v = c0 == 0 ? n0 : ccnt[(long)b * nchunk + min(ch, nch - 1)];
            const int n = ch < nch ? v : 0;
            const int inc = wave_incl_scan(n);
            if (lane == 63) s_w[wave] = inc;
            __syncthreads();
            int before = 0;
            for (int w = 0; w < wave; w++) before += s_w[w];
            if (ch < nch) {
                s_off[ch] = carry + before + inc - n;
                s_kc[ch] = 0;
            }
            carry += s_w[0] + s_w[1] + s_w[2] + s_w[3];
            __syncthreads();
        }
        if (tid == 0) s_off[nch] = carry;
        __syncthreads();
    }
    const int c = s_off[nch];  // the items inside the bin: >= need
    const u64 pm = (1ull << PB) - 1ull;
    // candidate i of the row: the last chunk whose offset is <= i, then its place in that chunk's run
    auto chunk_of = [&](int i) -> int {
        int lo = 0, hi = nch - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    auto entry = [&](int i) -> int2 {
        const int lo = chunk_of(i);
        return cr[(long)lo * SEL_CHUNK + (i - s_off[lo])];
    };
    auto key_of = [&](int2 e) -> u64 {
        return ((u64)(unsigned)(e.y - t.lo) << PB) | (pm - (u64)(unsigned)e.x);
    };
    const bool in_lds = c <= FCAP;
    if (in_lds)
        for (int i = tid; i < c; i += 256) s_key[i] = key_of(entry(i));
    __syncthreads();
    u64 prefix = 0, pmask = 0;
    if (t.need < c && in_lds && c <= 256) {
        // few candidates: the kept ones are those with fewer than `need` larger keys; the need-th largest key
        // becomes the threshold
        const u64 mine = tid < c ? s_key[tid] : 0ull;
        int rank = 0;
        for (int j = 0; j < c; j++) rank += s_key[j] > mine;
        if (tid < c && rank == t.need - 1) s_key[FCAP - 1] = mine;  // unique keys: exactly one thread
        __syncthreads();
        prefix = s_key[FCAP - 1];
        pmask = ~0ull;
        __syncthreads();
    } else if (t.need < c) {
        // the score offset is below 2^23 (the widest bin), so keys are below 2^(23 + PB)
        int krem = t.need;
        for (int shift = ((23 + PB - 1) / 8) * 8; shift >= 0; shift -= 8) {
            s_hist[tid] = 0;
            __syncthreads();
            for (int i = tid; i < c; i += 256) {
                const u64 k = in_lds ? s_key[i] : key_of(entry(i));
                if ((k & pmask) == prefix) atomicAdd(&s_hist[(unsigned)(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            // digit d: keys with a larger digit number fewer than krem, with d or larger at least krem
            const int d = 255 - tid;
            const int seg = (int)s_hist[d];
            int inc = wave_incl_scan(seg);
            if (lane == 63) s_w[wave] = inc;
            __syncthreads();
            int before = 0;
            for (int w = 0; w < wave; w++) before += s_w[w];
            inc += before;
            if (inc >= krem && inc - seg < krem) { s_pick[0] = d; s_pick[1] = inc - seg; s_pick[2] = seg; }
            __syncthreads();
            const int dd = s_pick[0], above = s_pick[1], cnt = s_pick[2];
            __syncthreads();
            prefix |= (u64)dd << shift;
            pmask |= 255ull << shift;
            krem -= above;
            if (cnt == krem) break;  // every key with this prefix is kept
        }
    }
    // kept candidates of the chunks before and in this workgroup's range: counts per chunk, and the bits of those
    // in its range
    for (int i = tid; i < FBW; i += 256) s_bm[i] = 0u;
    __syncthreads();
    for (int i = tid; i < s_off[cb]; i += 256) {
        const u64 k = in_lds ? s_key[i] : key_of(entry(i));
        if ((k & pmask) >= prefix) {
            const int ch = chunk_of(i);
            if (ch < ca) {
                atomicAdd(&s_kc[ch], 1);
            } else {
                const int item = (int)(pm - (k & pm));
                atomicOr(&s_bm[(item >> 5) - ca * (SEL_CHUNK / 32)], 1u << (item & 31));
            }
        }
    }
    __syncthreads();
    int kbefore = 0;
    for (int c0 = 0; c0 < ca; c0 += 256) kbefore += wave_sum_i(c0 + tid < ca ? s_kc[c0 + tid] : 0);
    if (lane == 0) s_w[wave] = kbefore;
    __syncthreads();
    const int base = abefore + s_w[0] + s_w[1] + s_w[2] + s_w[3];
    __syncthreads();
    // ordered compaction of this workgroup's words: thread tid owns word ca * 128 + tid
    if (tid < FBW) word |= s_bm[tid];
    const int cnt = __popc(word);
    const int inc = wave_incl_scan(cnt);
    if (lane == 63) s_w[wave] = inc;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; w++) before += s_w[w];
    const int tot = s_w[0] + s_w[1] + s_w[2] + s_w[3];
    int o = before + inc - cnt;
    // the items go to LDS in order, then every thread stores consecutive slots
    unsigned x = word;
    while (x) {
        const int bit = __ffs((int)x) - 1;
        x &= x - 1u;
        s_out[o++] = wi * 32 + bit;
    }
    __syncthreads();
    for (int i = tid; i < tot; i += 256) put(base + i, s_out[i]);
}

// ------------------------------------------------------------------ host side
static int max_len(const dl_pages &pg) { return pg.max_pages_per_seq * pg.page_size; }

void topk_ws_layout(Ws &w, const dl_pages &pg, TopkWs &t, int R, int pool)
{
    const long B = (long)pg.batch * R, Lmax = max_len(pg) / pool;  // one selection per row, over items
    const long nchunk = (Lmax + SEL_CHUNK - 1) / SEL_CHUNK;
    t.scores = w.take<int32_t>(B * Lmax);
    t.hist1 = w.take<unsigned>(B * NB1);
    t.hflag = w.take<unsigned long long>(pg.batch);
    t.bits = w.take<unsigned>(B * nchunk * (SEL_CHUNK / 32));
    t.cand = w.take<int2>(B * nchunk * SEL_CHUNK);
    t.ccnt = w.take<int32_t>(B * nchunk);
    t.acnt = w.take<int32_t>(B * nchunk);
    t.thr = w.take<Thr>(B);
}

// A number no earlier scoring launch of this process used: a counter from a start drawn once per process (mixed
// from the clock, the process id and an address), so that a flag left in reused memory is unlikely to match.
static unsigned long long next_epoch()
{
    static std::atomic<unsigned long long> n{0};
    static const unsigned long long base = [] {
        unsigned long long x = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
        x ^= (unsigned long long)getpid() << 32;
        x ^= (unsigned long long)(uintptr_t)&n;
        // splitmix64 finaliser
        x += 0x9E3779B97F4A7C15ull;
        x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
        x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
        return x ^ (x >> 31);
    }();
    const unsigned long long e = base + n.fetch_add(1);
    return e ? e : 1;
}

template <int NHG, int KCH>
static void launch_score(hipStream_t s, const int8_t *q, const int8_t *kp, const dl_pages &pg, int ps_shift, int HI,
                         int DI, const TopkWs &t, long Lmax, int R, int pool)
{
    const unsigned long long epoch = next_epoch();
#define DL_SCORE_R(R_)                                                                                              \
    if (R == R_) {                                                                                                  \
        constexpr int W = score_wpb(NHG, KCH, R_), P = W * 4 * 64; /* waves, positions per workgroup */            \
        const int nblk = (int)((Lmax + P - 1) / P);                                                                 \
        hipLaunchKernelGGL((k_index_score<NHG, KCH, R_>), dim3(nblk, pg.batch), dim3(W * 64), 0, s, q, kp,           \
                           pg.page_table, pg.seq_lens, pool, pg.max_pages_per_seq, ps_shift, HI, DI, t.scores, Lmax,  \
                           t.hist1, t.hflag, epoch, pg.key_layout == DL_LAYOUT_TILES);                              \
    }
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
    const long Lw = (long)nchunk * (SEL_CHUNK / 32);  // bitmap words per row
    const int PB = Lmax > 1 ? 32 - __builtin_clz((unsigned)(Lmax - 1)) : 1;  // bits of an item index
    if (nchunk > FCH) return fail(DL_ERR_UNSUPPORTED, "indexer: %ld items per row (<= %d)", Lmax, FCH * SEL_CHUNK);
    const int nhg = (HI + 15) / 16, kch = (DI + 63) / 64;
#define DL_SCORE_CASE(H_, K_) \
    if (nhg == H_ && kch == K_) launch_score<H_, K_>(s, q_idx, k_pool, pg, ps_shift, HI, DI, t, Lmax, R, pool); else
    DL_SCORE_CASE(1, 1) DL_SCORE_CASE(1, 2) DL_SCORE_CASE(1, 3) DL_SCORE_CASE(1, 4)
    DL_SCORE_CASE(2, 1) DL_SCORE_CASE(2, 2) DL_SCORE_CASE(2, 3) DL_SCORE_CASE(2, 4)
    DL_SCORE_CASE(3, 1) DL_SCORE_CASE(3, 2) DL_SCORE_CASE(3, 3) DL_SCORE_CASE(3, 4)
    DL_SCORE_CASE(4, 1) DL_SCORE_CASE(4, 2) DL_SCORE_CASE(4, 3) DL_SCORE_CASE(4, 4)
    return fail(DL_ERR_UNSUPPORTED, "indexer shape heads=%d dim=%d", HI, DI);
#undef DL_SCORE_CASE
    hipLaunchKernelGGL(k_sel_mark, dim3(nchunk, B), dim3(256), 0, s, t.scores, Lmax, pg.seq_lens, R, pool, top_k,
                       t.hist1, t.bits, Lw, t.cand, t.ccnt, t.acnt, nchunk, t.thr);
    // rows of at most top_k items are written in FCPW-chunk pieces too; with top_k above the longest row that is
    // up to top_k items
    const long span = std::max(Lmax, (long)top_k);
    const int gfin = (int)((span + FCPW * SEL_CHUNK - 1) / (FCPW * SEL_CHUNK));
    hipLaunchKernelGGL(k_sel_final, dim3(gfin, B), dim3(256), 0, s, t.scores, Lmax, pg.seq_lens, R, pool, top_k,
                       t.bits, Lw, t.cand, t.ccnt, t.acnt, nchunk, t.thr, PB, sel, sel_score);
    return hip_check("indexer_topk");
}

}  // namespace dl
