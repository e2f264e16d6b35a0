// Host-side construction of the 4-bit decode tables.
#pragma once

#include <stdint.h>

namespace qlora {

// Stored 4-bit types (values of qlora_qtype).
enum QType { kQNF4 = 0, kQINT4 = 1, kQFP4 = 2, kQTypes = 3 };

double normal_quantile(double p);
void build_codebook(float out[16]);

// The 16 fp32 decode values of a stored type, indexed by code.
void build_type_table(int qtype, float out[16]);

// The type's distinct values in ascending order with the code of each, and
// the code of the value 0 (codes never produced by the quantizer are left
// out: Int4's -8 and FP4's -0).
struct TypeLevels {
  int n;
  float level[16];
  uint32_t code[16];
  uint32_t zero_code;
};
void build_type_levels(int qtype, const float table[16], TypeLevels* out);

}  // namespace qlora
