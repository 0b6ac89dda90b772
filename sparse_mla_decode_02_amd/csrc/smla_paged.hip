// The paged-pool instances of the decode kernel and their launcher, built
// without the VGPR-form MFMA option of the rest of the library (see the note
// at smla_launch_paged_decode in smla.hip).
#define SMLA_PAGED_TU
#include "smla.hip"
