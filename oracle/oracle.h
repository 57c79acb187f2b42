/* Reference oracle for speculative sampling's verify-and-resample step.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark; never by the GPU library.  This
 * header belongs to the oracle alone and is not shared with the library.
 *
 * Layouts (host memory, row-major, V fastest):
 *   target_logits [B][K_max+1][V]   dtype ORACLE_F32 (float) or ORACLE_BF16
 *                                   (uint16 holding bfloat16 bits)
 *   draft_logits  [B][K_max][V]
 *   draft_tokens  [B][K_max]        int32
 *   per-row arrays [B] or NULL (NULL means "use the default_* scalar")
 * Outputs:
 *   accepted [B]  n in [0, K_b], or -1 for an error row
 *   out_tokens [B][K_max+1]  d_0..d_{n-1}, y, then -1
 *   row_status [B]  ORACLE_ST_* bits
 *   diag [B][K_max][2] (may be NULL)  (q_t(d_t), p_t(d_t)) in double; NaN
 *        where t >= K_b or the row is an error row
 *   flags [B] (may be NULL)  ORACLE_FL_* bits: decisions within 1e-6 of
 *        their boundary
 *   resid_mass [B] (may be NULL)  the mass S the final draw normalised by
 */
#ifndef SPEC_SAMPLING_ORACLE_H
#define SPEC_SAMPLING_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_PLAIN = 0, ORACLE_TOPK = 1, ORACLE_TOPP = 2, ORACLE_GREEDY = 3 };
enum { ORACLE_PURPOSE_ACCEPT = 0, ORACLE_PURPOSE_RESAMPLE = 1, ORACLE_PURPOSE_BONUS = 2 };

enum {
  ORACLE_ST_TOKEN = 1u << 0,         /* draft token outside [0, V)        */
  ORACLE_ST_NONFINITE = 1u << 1,     /* NaN or +inf in a used logit row   */
  ORACLE_ST_EMPTY = 1u << 2,         /* every logit of a used row is -inf */
  ORACLE_ST_ZERO_RESIDUAL = 1u << 3, /* residual had no mass: drew from q */
  ORACLE_ST_PZERO = 1u << 4,         /* a tested draft token had p = 0    */
  ORACLE_ST_PARAM = 1u << 6          /* invalid per-row parameter         */
};
#define ORACLE_ST_ERRORS (ORACLE_ST_TOKEN | ORACLE_ST_NONFINITE | ORACLE_ST_EMPTY | ORACLE_ST_PARAM)

enum { ORACLE_FL_ACCEPT = 1u << 0, ORACLE_FL_CDF = 1u << 1, ORACLE_FL_TOPP = 1u << 2 };

typedef struct {
  int32_t B, K_max, V, dtype;
  const void* target_logits;
  const void* draft_logits;
  const int32_t* draft_tokens;
  const int32_t* k_per_row;
  const uint8_t* mode;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  int32_t default_mode;
  float default_temperature;
  int32_t default_top_k;
  float default_top_p;
  uint64_t seed;
  uint64_t row_offset;
  int32_t* accepted;
  int32_t* out_tokens;
  uint32_t* row_status;
  double* diag;
  uint32_t* flags;
  double* resid_mass;
} OracleArgs;

void oracle_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out);
void oracle_philox_words(uint64_t seed, uint64_t n, const uint64_t* g, const uint32_t* t,
                         const uint32_t* purpose, uint32_t* out_words);
double oracle_uniform(uint64_t seed, uint64_t g, uint32_t t, uint32_t purpose);
uint32_t oracle_row_probs(const void* logits, int dtype, int V, int mode, float tau, int top_k,
                          float top_p, double* pi_out, double* topp_margin, int* n_keep);
int oracle_verify(const OracleArgs* a);

#ifdef __cplusplus
}
#endif
#endif
