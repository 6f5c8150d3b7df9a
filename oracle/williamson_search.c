/*
 * Search for Williamson matrices of order 43, from which the oracle builds a
 * Hadamard matrix of order 172 = 4*43 (test infrastructure; not product code).
 *
 * Why: the QuaRot paper (arXiv 2404.00456, "Hadamard background" paragraph)
 * factors a width d = 2^n * m and uses H_{2^n} (x) H_m with m the order of a
 * known Hadamard matrix from Sloane's list.  The Llama-2-7B FFN width
 * 11008 = 64 * 172 needs one of order 172.  The pages print none, so we
 * construct one here.
 *
 * Williamson's construction: four symmetric circulant +-1 matrices A, B, C, D
 * of odd order n with A^2 + B^2 + C^2 + D^2 = 4n I give the Hadamard matrix
 *     [  A  B  C  D ]
 *     [ -B  A -D  C ]
 *     [ -C  D  A -B ]
 *     [ -D -C  B  A ]
 * of order 4n.  For symmetric circulants the condition is that the periodic
 * autocorrelations (PAF) of the four first rows sum to zero at every shift
 * s = 1..(n-1)/2, equivalently that the four eigenvalue spectra satisfy
 * lam_A(k)^2 + lam_B(k)^2 + lam_C(k)^2 + lam_D(k)^2 = 4n for every k.
 *
 * Method: meet in the middle.  Sequences are enumerated over the orbits of a
 * multiplier subgroup G of Z_43^* that contains -1 (G = {+-1} is the full
 * symmetric search).  Each sequence must satisfy lam(k)^2 <= 4n (power
 * spectral density filter).  Row sums (a, b, c, d) must satisfy
 * a^2 + b^2 + c^2 + d^2 = 172 with all of them odd and positive (negating a
 * matrix keeps its square).  Pairs (A, B) are hashed by PAF_A + PAF_B and
 * pairs (C, D) look up -(PAF_C + PAF_D).  Any hit is verified exactly.
 *
 * Usage: williamson_search <subgroup generator g>   (g = 42 -> {+-1})
 * Prints the lexicographically smallest solution (by orbit masks) of the
 * first row-sum decomposition that has one, as four lines of 43 characters
 * '+'/'-'.  Generator 7 (an order-6 subgroup) finds one in well under a
 * second with row sums (5, 7, 7, 7).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define N 43
#define HALF 21
#define FOUR_N 172

typedef struct {
  uint32_t mask;
  int r;
  int8_t paf[HALF];
  float psd[HALF];
} seq_t;

static int orbit_of[N];
static int norb;

static void build_orbits(int g) {
  for (int i = 0; i < N; ++i) orbit_of[i] = -1;
  orbit_of[0] = 0;
  norb = 1;
  for (int i = 1; i < N; ++i) {
    if (orbit_of[i] >= 0) continue;
    /* orbit of i under <g, -1> */
    int x = i;
    for (int t = 0; t < 2 * N; ++t) {
      orbit_of[x] = norb;
      orbit_of[N - x] = norb;
      x = (x * g) % N;
    }
    ++norb;
  }
}

static void seq_from_mask(uint32_t mask, int *x) {
  for (int i = 0; i < N; ++i) x[i] = ((mask >> orbit_of[i]) & 1u) ? -1 : 1;
}

static double costab[HALF + 1][N];

static void init_costab(void) {
  for (int k = 0; k <= HALF; ++k)
    for (int i = 0; i < N; ++i) costab[k][i] = cos(2.0 * M_PI * (double)((i * k) % N) / N);
}

static void analyse(uint32_t mask, seq_t *s) {
  int x[N];
  seq_from_mask(mask, x);
  s->mask = mask;
  int r = 0;
  for (int i = 0; i < N; ++i) r += x[i];
  s->r = r;
  for (int sh = 1; sh <= HALF; ++sh) {
    int acc = 0;
    for (int i = 0; i < N; ++i) acc += x[i] * x[(i + sh) % N];
    s->paf[sh - 1] = (int8_t)acc;
  }
  for (int k = 1; k <= HALF; ++k) {
    double lam = 0.0;
    for (int i = 0; i < N; ++i) lam += x[i] * costab[k][i];
    s->psd[k - 1] = (float)(lam * lam);
  }
}

static int psd_ok(const seq_t *s) {
  for (int k = 0; k < HALF; ++k)
    if (s->psd[k] > FOUR_N + 1e-3f) return 0;
  return 1;
}

/* candidates per positive odd row sum */
static seq_t *cls[16];
static size_t ncls[16];

static uint64_t hash_key(const int8_t *v) {
  uint64_t h = 1469598103934665603ull;
  for (int i = 0; i < HALF; ++i) {
    h ^= (uint8_t)v[i];
    h *= 1099511628211ull;
  }
  return h ? h : 1;
}

typedef struct {
  uint64_t h;
  uint32_t ia, ib;
} slot_t;

static slot_t *table;
static size_t tcap;

static void tinsert(uint64_t h, uint32_t ia, uint32_t ib) {
  size_t p = h & (tcap - 1);
  while (table[p].h) p = (p + 1) & (tcap - 1);
  table[p].h = h;
  table[p].ia = ia;
  table[p].ib = ib;
}

static void print_seq(uint32_t mask) {
  int x[N];
  seq_from_mask(mask, x);
  for (int i = 0; i < N; ++i) putchar(x[i] > 0 ? '+' : '-');
  putchar('\n');
}

static int verify(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  int xs[4][N];
  seq_from_mask(a, xs[0]);
  seq_from_mask(b, xs[1]);
  seq_from_mask(c, xs[2]);
  seq_from_mask(d, xs[3]);
  for (int sh = 1; sh < N; ++sh) {
    int acc = 0;
    for (int m = 0; m < 4; ++m)
      for (int i = 0; i < N; ++i) acc += xs[m][i] * xs[m][(i + sh) % N];
    if (acc != 0) return 0;
  }
  return 1;
}

static int run_decomp(int ra, int rb, int rc, int rd) {
  seq_t *A = cls[ra], *B = cls[rb], *C = cls[rc], *D = cls[rd];
  size_t na = ncls[ra], nb = ncls[rb], nc = ncls[rc], nd = ncls[rd];
  fprintf(stderr, "decomp (%d,%d,%d,%d): |A|=%zu |B|=%zu |C|=%zu |D|=%zu\n", ra, rb, rc, rd,
          na, nb, nc, nd);
  if (!na || !nb || !nc || !nd) return 0;
  /* count surviving AB pairs */
  size_t cnt = 0;
  for (size_t i = 0; i < na; ++i)
    for (size_t j = (ra == rb ? i : 0); j < nb; ++j) {
      int ok = 1;
      for (int k = 0; k < HALF && ok; ++k) ok = A[i].psd[k] + B[j].psd[k] <= FOUR_N + 1e-3f;
      cnt += ok;
    }
  fprintf(stderr, "  AB pairs surviving: %zu\n", cnt);
  tcap = 1;
  while (tcap < 2 * cnt + 16) tcap <<= 1;
  table = (slot_t *)calloc(tcap, sizeof(slot_t));
  if (!table) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  for (size_t i = 0; i < na; ++i)
    for (size_t j = (ra == rb ? i : 0); j < nb; ++j) {
      int ok = 1;
      for (int k = 0; k < HALF && ok; ++k) ok = A[i].psd[k] + B[j].psd[k] <= FOUR_N + 1e-3f;
      if (!ok) continue;
      int8_t key[HALF];
      for (int k = 0; k < HALF; ++k) key[k] = (int8_t)(A[i].paf[k] + B[j].paf[k]);
      tinsert(hash_key(key), (uint32_t)i, (uint32_t)j);
    }
  int found = 0;
  uint32_t sol[4] = {0, 0, 0, 0};
#pragma omp parallel for schedule(dynamic, 16)
  for (size_t i = 0; i < nc; ++i) {
    for (size_t j = (rc == rd ? i : 0); j < nd; ++j) {
      int ok = 1;
      for (int k = 0; k < HALF && ok; ++k) ok = C[i].psd[k] + D[j].psd[k] <= FOUR_N + 1e-3f;
      if (!ok) continue;
      int8_t key[HALF];
      for (int k = 0; k < HALF; ++k) key[k] = (int8_t)(-(C[i].paf[k] + D[j].paf[k]));
      uint64_t h = hash_key(key);
      size_t p = h & (tcap - 1);
      while (table[p].h) {
        if (table[p].h == h) {
          const seq_t *a = &A[table[p].ia], *b = &B[table[p].ib];
          if (verify(a->mask, b->mask, C[i].mask, D[j].mask)) {
            /* keep the lexicographically smallest (A, B, C, D) mask tuple so
               that the output does not depend on thread scheduling */
            uint32_t cand[4] = {a->mask, b->mask, C[i].mask, D[j].mask};
#pragma omp critical
            {
              int better = !found;
              for (int m = 0; m < 4 && !better; ++m) {
                if (cand[m] != sol[m]) {
                  better = cand[m] < sol[m];
                  break;
                }
              }
              if (better) memcpy(sol, cand, sizeof(sol));
              found = 1;
            }
          }
        }
        p = (p + 1) & (tcap - 1);
      }
    }
  }
  free(table);
  if (found) {
    for (int m = 0; m < 4; ++m) print_seq(sol[m]);
    fflush(stdout);
  }
  return found;
}

int main(int argc, char **argv) {
  int g = argc > 1 ? atoi(argv[1]) : 42;
  build_orbits(g);
  init_costab();
  fprintf(stderr, "generator %d: %d orbits\n", g, norb);
  if (norb > 30) return 1;
  uint32_t total = 1u << norb;
  for (int r = 0; r < 16; ++r) {
    cls[r] = NULL;
    ncls[r] = 0;
  }
  size_t cap[16] = {0};
  for (uint32_t m = 0; m < total; ++m) {
    seq_t s;
    analyse(m, &s);
    if (s.r <= 0 || s.r > 13) continue;
    if (!psd_ok(&s)) continue;
    if (ncls[s.r] == cap[s.r]) {
      cap[s.r] = cap[s.r] ? 2 * cap[s.r] : 1024;
      cls[s.r] = (seq_t *)realloc(cls[s.r], cap[s.r] * sizeof(seq_t));
    }
    cls[s.r][ncls[s.r]++] = s;
  }
  /* all ways to write 172 as a sum of four positive odd squares (sorted) */
  const int dec[][4] = {{1, 1, 1, 13}, {1, 1, 7, 11}, {1, 3, 9, 9}, {1, 5, 5, 11}, {5, 7, 7, 7}};
  for (int t = 0; t < 5; ++t) {
    /* hash the pair with the fewest candidates */
    if (run_decomp(dec[t][0], dec[t][1], dec[t][2], dec[t][3])) return 0;
  }
  fprintf(stderr, "no solution with this orbit structure\n");
  return 3;
}
