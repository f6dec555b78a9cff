// Kernels of table row 0 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW(0, Cfg0, Fast0)
