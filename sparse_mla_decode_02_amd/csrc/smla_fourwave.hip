// The contiguous-cache instances of the four-wave decode kernel and their
// launcher, built without the instruction-level-parallelism scheduler of the
// library's main unit (see the note at smla_launch_fourwave_decode in
// smla.hip).
#define SMLA_FOURWAVE_TU
#include "smla.hip"
